/*
 * decode_c.c - a plain C11 caller of the LoopVQ decode path, using only
 * loopvq.h and the HIP runtime API (no Python, no torch).
 *
 * Usage: decode_c DIR
 *   DIR/args.txt   whitespace-separated "name value" pairs: the loopvq_config
 *                  fields under their struct names, plus layer, loop, batch,
 *                  max_pages_per_seq, max_seq_len, num_splits, num_pages,
 *                  pool_offset and pool_slice_bytes (the byte range of this
 *                  (layer, loop group) inside the whole pool), softmax_scale,
 *                  has_rot, and optionally encode (0 or 1) and n_rows
 *   DIR/q.bin, lens.bin, bt.bin, cbk.bin, cbv.bin, kp.bin, vp.bin, kr.bin,
 *   vr.bin [, rot.bin]   raw little-endian arrays in the layouts loopvq.h states
 *                  (canonical codebooks, one (layer, loop step) of windows)
 *   without encode: DIR/pool.bin, the packed pages of the pool range
 *   with encode 1:  DIR/src_k.bin, src_v.bin (bf16 [G][n_rows][Hkv][d], the
 *                  loop group's G loop steps of every row to encode),
 *                  seq_id.bin and vq_pos.bin (int32 [n_rows]); the rows are
 *                  encoded into a zeroed pool first, and the pool range is
 *                  written to DIR/pool_out.bin
 * Writes DIR/out.bin (fp32 [B][Hq][d]) and DIR/lse.bin (fp32 [B][Hq]).
 *
 * The program owns every device buffer, as the library's conventions require:
 * it sizes them with loopvq_layout_query and loopvq_decode_attn_workspace,
 * prepares both codebook kinds (and their norms) with loopvq_codebook_prepare,
 * optionally encodes K and V rows with loopvq_encode, runs one decode launch,
 * and also checks that a host-detectable mistake (batch 0) returns
 * LOOPVQ_ERR_INVALID_ARG with a message before any HIP call.
 * Exit status 0 on success, 1 on any failure (with a message on stderr).
 */
#include <hip/hip_runtime_api.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "loopvq.h"

#define FAIL(...)                         \
  do {                                    \
    fprintf(stderr, "decode_c: ");        \
    fprintf(stderr, __VA_ARGS__);         \
    fprintf(stderr, "\n");                \
    exit(1);                              \
  } while (0)

#define HIP_OK(call)                                                              \
  do {                                                                            \
    hipError_t e_ = (call);                                                       \
    if (e_ != hipSuccess) FAIL("%s failed: %s", #call, hipGetErrorString(e_));    \
  } while (0)

#define LVQ_OK(call)                                                              \
  do {                                                                            \
    loopvq_status s_ = (call);                                                    \
    if (s_ != LOOPVQ_OK)                                                          \
      FAIL("%s returned %s: %s", #call, loopvq_status_string(s_), loopvq_last_error()); \
  } while (0)

enum { MAX_ARGS = 64 };
static char arg_name[MAX_ARGS][64];
static double arg_val[MAX_ARGS];
static int n_args;

static void read_args(const char* dir) {
  char path[4096];
  snprintf(path, sizeof path, "%s/args.txt", dir);
  FILE* f = fopen(path, "r");
  if (!f) FAIL("cannot open %s", path);
  while (n_args < MAX_ARGS && fscanf(f, "%63s %lf", arg_name[n_args], &arg_val[n_args]) == 2) n_args++;
  fclose(f);
}

static int find_arg(const char* name) {
  for (int i = 0; i < n_args; i++)
    if (strcmp(arg_name[i], name) == 0) return i;
  return -1;
}

static double arg(const char* name) {
  const int i = find_arg(name);
  if (i < 0) FAIL("args.txt lacks %s", name);
  return arg_val[i];
}

static double arg_or(const char* name, double fallback) {
  const int i = find_arg(name);
  return i < 0 ? fallback : arg_val[i];
}

/* Read DIR/name into a new host buffer of exactly `bytes` bytes (the file must match). */
static void* read_file(const char* dir, const char* name, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "rb");
  if (!f) FAIL("cannot open %s", path);
  fseek(f, 0, SEEK_END);
  long size = ftell(f);
  fseek(f, 0, SEEK_SET);
  if (size < 0 || (size_t)size != bytes) FAIL("%s holds %ld bytes, expected %zu", path, size, bytes);
  void* p = malloc(bytes ? bytes : 1);
  if (!p) FAIL("out of host memory");
  if (bytes && fread(p, 1, bytes, f) != bytes) FAIL("short read of %s", path);
  fclose(f);
  return p;
}

static void write_file(const char* dir, const char* name, const void* p, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "wb");
  if (!f) FAIL("cannot create %s", path);
  if (fwrite(p, 1, bytes, f) != bytes) FAIL("short write of %s", path);
  fclose(f);
}

/* Copy a host file to a new device buffer (at least 16 bytes, so that every pointer is valid). */
static void* upload(const char* dir, const char* name, size_t bytes) {
  void* h = read_file(dir, name, bytes);
  void* d = NULL;
  HIP_OK(hipMalloc(&d, bytes > 16 ? bytes : 16));
  if (bytes) HIP_OK(hipMemcpy(d, h, bytes, hipMemcpyHostToDevice));
  free(h);
  return d;
}

int main(int argc, char** argv) {
  if (argc != 2) FAIL("usage: decode_c DIR");
  const char* dir = argv[1];
  read_args(dir);

  loopvq_config cfg;
  cfg.num_layers = (int32_t)arg("num_layers");
  cfg.num_loops = (int32_t)arg("num_loops");
  cfg.loop_group = (int32_t)arg("loop_group");
  cfg.num_q_heads = (int32_t)arg("num_q_heads");
  cfg.num_kv_heads = (int32_t)arg("num_kv_heads");
  cfg.head_dim = (int32_t)arg("head_dim");
  cfg.chans_per_group = (int32_t)arg("chans_per_group");
  cfg.index_bits = (int32_t)arg("index_bits");
  cfg.prefix_tokens = (int32_t)arg("prefix_tokens");
  cfg.recent_tokens = (int32_t)arg("recent_tokens");
  cfg.page_tokens = (int32_t)arg("page_tokens");
  cfg.codebook_per_loop_group = (int32_t)arg("codebook_per_loop_group");
  LVQ_OK(loopvq_config_check(&cfg));

  const int32_t batch = (int32_t)arg("batch");
  const int32_t max_pages = (int32_t)arg("max_pages_per_seq");
  const int32_t max_len = (int32_t)arg("max_seq_len");
  const int32_t num_splits = (int32_t)arg("num_splits");
  const int64_t num_pages = (int64_t)arg("num_pages");
  const int64_t pool_offset = (int64_t)arg("pool_offset");
  const int64_t pool_slice = (int64_t)arg("pool_slice_bytes");
  const int has_rot = (int)arg("has_rot");
  const int encode = (int)arg_or("encode", 0.0);
  const int64_t Hq = cfg.num_q_heads, d = cfg.head_dim;

  loopvq_layout lay;
  LVQ_OK(loopvq_layout_query(&cfg, batch, num_pages, &lay));
  if (pool_offset < 0 || pool_slice < 0 || pool_offset + pool_slice > lay.pool_bytes)
    FAIL("pool slice [%lld, %lld) outside the %lld-byte pool", (long long)pool_offset,
         (long long)(pool_offset + pool_slice), (long long)lay.pool_bytes);
  printf("decode_c: %.3f bits per element, pool %lld bytes, page %lld bytes\n", loopvq_bits_per_elem(&cfg),
         (long long)lay.pool_bytes, (long long)lay.page_bytes);

  /* inputs */
  void* d_q = upload(dir, "q.bin", (size_t)(batch * Hq * d * 2));
  void* d_lens = upload(dir, "lens.bin", (size_t)batch * 4);
  void* d_bt = upload(dir, "bt.bin", (size_t)batch * max_pages * 4);
  void* d_cb[2] = {upload(dir, "cbk.bin", (size_t)lay.codebook_elems * 2),
                   upload(dir, "cbv.bin", (size_t)lay.codebook_elems * 2)};
  void* d_kp = upload(dir, "kp.bin", (size_t)lay.prefix_elems * 2);
  void* d_vp = upload(dir, "vp.bin", (size_t)lay.prefix_elems * 2);
  void* d_kr = upload(dir, "kr.bin", (size_t)lay.recent_elems * 2);
  void* d_vr = upload(dir, "vr.bin", (size_t)lay.recent_elems * 2);
  void* d_rot = has_rot ? upload(dir, "rot.bin", (size_t)(d * d * 4)) : NULL;

  /* the whole pool, zeroed (unwritten slots must be zero) */
  void* d_pool = NULL;
  HIP_OK(hipMalloc(&d_pool, (size_t)lay.pool_bytes));
  HIP_OK(hipMemset(d_pool, 0, (size_t)lay.pool_bytes));
  if (!encode) {   /* the slice the caller packed */
    void* h = read_file(dir, "pool.bin", (size_t)pool_slice);
    if (pool_slice) HIP_OK(hipMemcpy((char*)d_pool + pool_offset, h, (size_t)pool_slice, hipMemcpyHostToDevice));
    free(h);
  }

  /* decode-side codebook copies and squared norms, one per kind */
  void* d_prep[2];
  void* d_norm[2];
  for (int kind = 0; kind < 2; kind++) {
    HIP_OK(hipMalloc(&d_prep[kind], (size_t)lay.codebook_elems * 2));
    HIP_OK(hipMalloc(&d_norm[kind], (size_t)lay.norms_elems * 4));
    LVQ_OK(loopvq_codebook_prepare(&cfg, (const uint16_t*)d_cb[kind], (uint16_t*)d_prep[kind], (float*)d_norm[kind],
                                   NULL));
  }

  /* optionally: encode the rows of the loop group into the pool, K then V */
  void *d_src[2] = {NULL, NULL}, *d_seq = NULL, *d_pos = NULL;
  if (encode) {
    const int32_t n_rows = (int32_t)arg("n_rows");
    const int64_t G = cfg.loop_group, Hkv = cfg.num_kv_heads;
    const size_t plane = (size_t)(n_rows * Hkv * d);
    d_src[0] = upload(dir, "src_k.bin", (size_t)G * plane * 2);
    d_src[1] = upload(dir, "src_v.bin", (size_t)G * plane * 2);
    d_seq = upload(dir, "seq_id.bin", (size_t)n_rows * 4);
    d_pos = upload(dir, "vq_pos.bin", (size_t)n_rows * 4);
    for (int kind = 0; kind < 2; kind++) {
      loopvq_encode_args ea;
      memset(&ea, 0, sizeof ea);
      ea.layer = (int32_t)arg("layer");
      ea.loop_group = (int32_t)arg("loop") / cfg.loop_group;
      ea.kind = kind;
      ea.n_tokens = n_rows;
      ea.src = (const uint16_t*)d_src[kind];
      ea.stride_loop = (int64_t)plane;
      ea.stride_token = Hkv * d;
      ea.stride_head = d;
      ea.seq_id = (const int32_t*)d_seq;
      ea.vq_pos = (const int32_t*)d_pos;
      ea.block_table = (const int32_t*)d_bt;
      ea.batch = batch;
      ea.max_pages_per_seq = max_pages;
      ea.num_pages = num_pages;
      ea.cb = (const uint16_t*)d_cb[kind];
      ea.cb_norms = (const float*)d_norm[kind];
      ea.pool = (uint8_t*)d_pool;
      LVQ_OK(loopvq_encode(&cfg, &ea, NULL));
    }
    HIP_OK(hipDeviceSynchronize());
    void* h = malloc(pool_slice ? (size_t)pool_slice : 1);
    if (!h) FAIL("out of host memory");
    if (pool_slice) HIP_OK(hipMemcpy(h, (char*)d_pool + pool_offset, (size_t)pool_slice, hipMemcpyDeviceToHost));
    write_file(dir, "pool_out.bin", h, (size_t)pool_slice);
    free(h);
  }

  /* outputs and workspace */
  size_t out_bytes = (size_t)(batch * Hq * d * 4), lse_bytes = (size_t)(batch * Hq * 4);
  void *d_out = NULL, *d_lse = NULL, *d_ws = NULL;
  HIP_OK(hipMalloc(&d_out, out_bytes));
  HIP_OK(hipMalloc(&d_lse, lse_bytes));
  size_t ws_bytes = 0;
  LVQ_OK(loopvq_decode_attn_workspace(&cfg, batch, max_len, &ws_bytes));
  if (num_splits > 1) {
    size_t explicit_bytes = (size_t)num_splits * (size_t)(batch * Hq * (d + 4) * 4);
    if (explicit_bytes > ws_bytes) ws_bytes = explicit_bytes;
  }
  HIP_OK(hipMalloc(&d_ws, ws_bytes > 16 ? ws_bytes : 16));

  loopvq_decode_args a;
  memset(&a, 0, sizeof a);
  a.layer = (int32_t)arg("layer");
  a.loop = (int32_t)arg("loop");
  a.batch = batch;
  a.max_pages_per_seq = max_pages;
  a.max_seq_len = max_len;
  a.num_splits = num_splits;
  a.num_pages = num_pages;
  a.q = (const uint16_t*)d_q;
  a.seq_lens = (const int32_t*)d_lens;
  a.block_table = (const int32_t*)d_bt;
  a.pool = (const uint8_t*)d_pool;
  a.cb_k_prep = (const uint16_t*)d_prep[0];
  a.cb_v_prep = (const uint16_t*)d_prep[1];
  a.k_prefix = (const uint16_t*)d_kp;
  a.v_prefix = (const uint16_t*)d_vp;
  a.k_recent = (const uint16_t*)d_kr;
  a.v_recent = (const uint16_t*)d_vr;
  a.rot = (const float*)d_rot;
  a.softmax_scale = (float)arg("softmax_scale");
  a.out = (float*)d_out;
  a.lse = (float*)d_lse;

  /* a host-detectable mistake is refused before any HIP call, with a message */
  {
    loopvq_decode_args bad = a;
    bad.batch = 0;
    loopvq_status s = loopvq_decode_attn(&cfg, &bad, d_ws, ws_bytes, NULL);
    if (s != LOOPVQ_ERR_INVALID_ARG || loopvq_last_error()[0] == '\0')
      FAIL("batch 0 returned %d (\"%s\"), expected LOOPVQ_ERR_INVALID_ARG with a message", s, loopvq_last_error());
  }

  LVQ_OK(loopvq_decode_attn(&cfg, &a, d_ws, ws_bytes, NULL));
  HIP_OK(hipDeviceSynchronize());

  void* h_out = malloc(out_bytes);
  void* h_lse = malloc(lse_bytes);
  if (!h_out || !h_lse) FAIL("out of host memory");
  HIP_OK(hipMemcpy(h_out, d_out, out_bytes, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(h_lse, d_lse, lse_bytes, hipMemcpyDeviceToHost));
  write_file(dir, "out.bin", h_out, out_bytes);
  write_file(dir, "lse.bin", h_lse, lse_bytes);
  free(h_out);
  free(h_lse);

  void* bufs[] = {d_q, d_lens, d_bt, d_cb[0], d_cb[1], d_kp, d_vp, d_kr, d_vr, d_rot, d_pool, d_prep[0],
                  d_prep[1], d_norm[0], d_norm[1], d_src[0], d_src[1], d_seq, d_pos, d_out, d_lse, d_ws};
  for (size_t i = 0; i < sizeof bufs / sizeof bufs[0]; i++)
    if (bufs[i]) HIP_OK(hipFree(bufs[i]));
  printf("decode_c: ok\n");
  return 0;
}
