// C ABI of the LoopVQ library: argument validation, layout arithmetic, split planning
// and kernel launches.  Every check runs before any HIP call, so a rejected call has
// no side effect; the only state is a thread-local error string.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/loopvq.h"
#include "lvq_common.h"

namespace {

thread_local char g_err[512] = "";

loopvq_status fail(loopvq_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

loopvq_status ok() {
  g_err[0] = '\0';
  return LOOPVQ_OK;
}

bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

int ilog2(int64_t v) {
  int r = 0;
  while ((int64_t(1) << r) < v) ++r;
  return r;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

loopvq_status check_config(const loopvq_config* c) {
  if (!c) return fail(LOOPVQ_ERR_INVALID_ARG, "config is NULL");
  if (c->num_layers < 1 || c->num_loops < 1 || c->loop_group < 1)
    return fail(LOOPVQ_ERR_INVALID_ARG, "num_layers, num_loops and loop_group must be >= 1");
  if (c->num_loops % c->loop_group)
    return fail(LOOPVQ_ERR_INVALID_ARG, "num_loops (%d) must be a multiple of loop_group (%d)", c->num_loops,
                c->loop_group);
  if (c->num_q_heads < 1 || c->num_kv_heads < 1 || c->num_q_heads % c->num_kv_heads)
    return fail(LOOPVQ_ERR_INVALID_ARG, "num_q_heads must be a positive multiple of num_kv_heads");
  if (c->head_dim < 1 || c->chans_per_group < 1 || c->head_dim % c->chans_per_group)
    return fail(LOOPVQ_ERR_INVALID_ARG, "head_dim must be a positive multiple of chans_per_group");
  if ((c->head_dim / c->chans_per_group) % 4)
    return fail(LOOPVQ_ERR_INVALID_ARG, "head_dim / chans_per_group must be a multiple of 4");
  if (c->index_bits < 1 || c->index_bits > 16) return fail(LOOPVQ_ERR_INVALID_ARG, "index_bits must be in [1, 16]");
  if (c->prefix_tokens < 0 || c->recent_tokens < 0)
    return fail(LOOPVQ_ERR_INVALID_ARG, "prefix_tokens and recent_tokens must be >= 0");
  if (c->page_tokens < 64 || !is_pow2(c->page_tokens))
    return fail(LOOPVQ_ERR_INVALID_ARG, "page_tokens must be a power of two >= 64");
  if (c->codebook_per_loop_group != 0 && c->codebook_per_loop_group != 1)
    return fail(LOOPVQ_ERR_INVALID_ARG, "codebook_per_loop_group must be 0 or 1");
  return LOOPVQ_OK;
}

// Variants the kernels are built for.
loopvq_status check_supported(const loopvq_config* c) {
  const int ng = c->head_dim / c->chans_per_group;
  if (c->index_bits != 8) return fail(LOOPVQ_ERR_UNSUPPORTED, "kernels are built for index_bits = 8 only");
  const int E = c->chans_per_group * c->loop_group;
  const bool okg = c->loop_group == 4 || (c->loop_group == 2 && c->chans_per_group == 8) ||
                   (c->loop_group == 8 && c->chans_per_group == 4);
  if (!okg)
    return fail(LOOPVQ_ERR_UNSUPPORTED,
                "kernels are built for (c, G) in {(4, 4), (8, 4), (8, 2), (4, 8)}; got (%d, %d), sub-vector length %d",
                c->chans_per_group, c->loop_group, E);
  const bool okv = (c->chans_per_group == 4 && (ng == 16 || ng == 32)) || (c->chans_per_group == 8 && ng == 16);
  if (!okv)
    return fail(LOOPVQ_ERR_UNSUPPORTED, "kernels are built for (c, d) in {(4, 64), (4, 128), (8, 128)}; got (%d, %d)",
                c->chans_per_group, c->head_dim);
  return LOOPVQ_OK;
}

struct Sizes {
  int ng, J, Jcb, K, E;
  int64_t tile_bytes, kind_bytes, page_bytes;
};

Sizes sizes_of(const loopvq_config* c) {
  Sizes s;
  s.ng = c->head_dim / c->chans_per_group;
  s.J = c->num_loops / c->loop_group;
  s.Jcb = c->codebook_per_loop_group ? s.J : 1;
  s.K = 1 << c->index_bits;
  s.E = c->chans_per_group * c->loop_group;
  s.tile_bytes = 2 * int64_t(c->index_bits);
  s.kind_bytes = int64_t(c->page_tokens / 4) * (s.ng / 4) * s.tile_bytes;
  s.page_bytes = 2 * s.kind_bytes;
  return s;
}

// Tokens per wave tile of the decode kernel (1 KB of 8-bit indices).
int decode_tile_tokens(const loopvq_config* c) { return 256 / ((c->head_dim / c->chans_per_group) / 4); }

// Fewest splits the decode kernel accepts: one split covers at most 2048 tiles at NG=32
// (16 waves x 128) or 1024 at NG=16 (8 waves x 128) -- the page ids a wave keeps in two
// VGPRs -- i.e. at most 65536 vector-quantized tokens, so the 64-bit value histogram (each
// token adds at most 2^47) cannot overflow.
int min_splits(const loopvq_config* c, int32_t max_seq_len) {
  const int64_t n_vq = std::max<int64_t>(0, int64_t(max_seq_len) - c->prefix_tokens - c->recent_tokens);
  const int64_t tiles = (n_vq + decode_tile_tokens(c) - 1) / decode_tile_tokens(c);
  const int64_t max_tiles = (c->head_dim / c->chans_per_group) == 32 ? 2048 : 1024;
  return (int)std::max<int64_t>(1, (tiles + max_tiles - 1) / max_tiles);
}

int plan_splits(const loopvq_config* c, int32_t batch, int32_t max_seq_len) {
  const int64_t Q = int64_t(batch) * c->num_q_heads;
  const int64_t n_vq = std::max<int64_t>(0, int64_t(max_seq_len) - c->prefix_tokens - c->recent_tokens);
  const int64_t n_win = std::min<int64_t>(max_seq_len, int64_t(c->prefix_tokens) + c->recent_tokens);
  const int64_t tiles = (n_vq + decode_tile_tokens(c) - 1) / decode_tile_tokens(c);
  // work in 2 KB index tiles (1 KB of K and of V indices); a bf16 window row moves 4 d bytes
  const int64_t work = tiles + (n_win * 4 * c->head_dim + 2047) / 2048;
  const int64_t slots = (c->head_dim / c->chans_per_group) == 32 ? 256 : 512;  // resident workgroups
  int64_t S = Q >= slots ? 1 : (slots + Q - 1) / Q;
  const int64_t max_by_work = std::max<int64_t>(1, work / 32);   // >= 32 tiles of work per split
  S = std::min(S, max_by_work);
  S = std::max<int64_t>(S, min_splits(c, max_seq_len));
  return (int)std::max<int64_t>(1, std::min<int64_t>(S, 256));
}

// Fields of an encode launch that depend only on the config and the pool.
lvq::EncodeParams encode_params(const loopvq_config* cfg, const Sizes& z, int32_t batch, int32_t max_pages,
                                int64_t num_pages) {
  lvq::EncodeParams p{};
  p.L = cfg->num_layers;
  p.J = z.J;
  p.Jcb = z.Jcb;
  p.T = cfg->num_loops;
  p.Hkv = cfg->num_kv_heads;
  p.NG = z.ng;
  p.G = cfg->loop_group;
  p.pt_shift = ilog2(cfg->page_tokens);
  p.max_pages = max_pages;
  p.batch = batch;
  p.num_pages = num_pages;
  p.page_bytes = z.page_bytes;
  p.kind_bytes = z.kind_bytes;
  p.head_stride = num_pages * z.page_bytes;
  return p;
}

// Row partition of the Lloyd sums kernel: one 1024-thread workgroup per CU (its fp64
// accumulator fills most of the LDS), so aim at 256 workgroups, with at least 2048 rows each.
struct LloydPlan {
  int chunks_a, rows_a;
  size_t sums_doubles, dist_doubles, w_doubles;
  size_t bytes() const { return (sums_doubles + dist_doubles + w_doubles) * sizeof(double); }
};

LloydPlan lloyd_plan(const loopvq_config* cfg, const Sizes& z, int32_t n) {
  LloydPlan pl;
  const int per_chunk = cfg->num_kv_heads * cfg->loop_group * (cfg->head_dim / 64);
  const int64_t by_rows = std::max<int64_t>(1, (int64_t(n) + 2047) / 2048);
  pl.chunks_a = (int)std::max<int64_t>(1, std::min<int64_t>((256 + per_chunk - 1) / per_chunk, by_rows));
  pl.rows_a = (int)((int64_t(n) + pl.chunks_a - 1) / pl.chunks_a);
  const size_t hk = size_t(pl.chunks_a) * cfg->num_kv_heads;
  pl.sums_doubles = hk * cfg->loop_group * cfg->head_dim * z.K;
  pl.dist_doubles = hk * cfg->loop_group * z.ng;
  pl.w_doubles = hk * z.ng * z.K;
  return pl;
}

loopvq_status check_lloyd(const loopvq_config* cfg, const loopvq_lloyd_args* a) {
  loopvq_status s = check_config(cfg);
  if (s) return s;
  if (!a) return fail(LOOPVQ_ERR_INVALID_ARG, "args is NULL");
  if ((s = check_supported(cfg))) return s;
  const Sizes z = sizes_of(cfg);
  if (a->layer < 0 || a->layer >= cfg->num_layers) return fail(LOOPVQ_ERR_INVALID_ARG, "layer out of range");
  if (a->cb_set < 0 || a->cb_set >= z.Jcb)
    return fail(LOOPVQ_ERR_INVALID_ARG, "cb_set %d out of range [0, %d)", a->cb_set, z.Jcb);
  if (a->n_samples < 0) return fail(LOOPVQ_ERR_INVALID_ARG, "n_samples must be >= 0");
  if (!a->src || !a->weight || !a->cb || !a->cb_norms || !a->assign || !a->workspace)
    return fail(LOOPVQ_ERR_INVALID_ARG, "src, weight, cb, cb_norms, assign and workspace must not be NULL");
  if (!aligned(a->src, 16) || a->stride_loop % 8 || a->stride_token % 8 || a->stride_head % 8)
    return fail(LOOPVQ_ERR_MISALIGNED, "src must be 16-byte aligned and its strides multiples of 8 elements");
  if (!aligned(a->weight, 16) || !aligned(a->assign, 16) || !aligned(a->cb, 16) || !aligned(a->cb_norms, 16) ||
      !aligned(a->workspace, 16) || (a->cluster_weight && !aligned(a->cluster_weight, 8)) ||
      (a->distortion && !aligned(a->distortion, 8)) || (a->rerank_count && !aligned(a->rerank_count, 8)))
    return fail(LOOPVQ_ERR_MISALIGNED, "weight, assign, cb, cb_norms and workspace must be 16-byte aligned, the "
                                       "optional outputs 8-byte aligned");
  const size_t need = lloyd_plan(cfg, z, a->n_samples).bytes();
  if (a->workspace_bytes < need) return fail(LOOPVQ_ERR_WORKSPACE, "workspace too small: %zu bytes needed", need);
  return LOOPVQ_OK;
}

// Checks of a decode call (every one before any HIP call) and its launch parameters; the split
// workspace is the caller's business: *need bytes of it, placed in p->ws.
loopvq_status decode_setup(const loopvq_config* cfg, const loopvq_decode_args* a, lvq::DecodeParams* out,
                           size_t* need_out) {
  loopvq_status s = check_config(cfg);
  if (s) return s;
  if (!a) return fail(LOOPVQ_ERR_INVALID_ARG, "args is NULL");
  if ((s = check_supported(cfg))) return s;
  const Sizes z = sizes_of(cfg);
  if (a->layer < 0 || a->layer >= cfg->num_layers) return fail(LOOPVQ_ERR_INVALID_ARG, "layer out of range");
  if (a->loop < 0 || a->loop >= cfg->num_loops) return fail(LOOPVQ_ERR_INVALID_ARG, "loop out of range");
  if (a->batch < 1) return fail(LOOPVQ_ERR_INVALID_ARG, "batch must be >= 1");
  if (a->max_seq_len < 1) return fail(LOOPVQ_ERR_INVALID_ARG, "max_seq_len must be >= 1");
  if (a->num_splits < 0 || a->num_splits > 256) return fail(LOOPVQ_ERR_INVALID_ARG, "num_splits must be in [0, 256]");
  if (int64_t(a->batch) * cfg->num_q_heads * 256 > (int64_t(1) << 31) - 1)
    return fail(LOOPVQ_ERR_INVALID_ARG, "batch * num_q_heads too large");
  if (!a->q || !a->seq_lens || !a->out) return fail(LOOPVQ_ERR_INVALID_ARG, "q, seq_lens and out must not be NULL");
  const bool can_vq = int64_t(a->max_seq_len) > int64_t(cfg->prefix_tokens) + cfg->recent_tokens;
  if (can_vq) {
    if (!a->block_table || !a->pool || !a->cb_k_prep || !a->cb_v_prep)
      return fail(LOOPVQ_ERR_INVALID_ARG, "block_table, pool and prepared codebooks must not be NULL");
    if (a->max_pages_per_seq < 1 || a->num_pages < 1)
      return fail(LOOPVQ_ERR_INVALID_ARG, "max_pages_per_seq and num_pages must be >= 1");
    if (int64_t(a->max_pages_per_seq) * cfg->page_tokens > INT32_MAX)
      return fail(LOOPVQ_ERR_INVALID_ARG, "max_pages_per_seq * page_tokens must stay below 2^31");
    if (!aligned(a->pool, 16) || !aligned(a->cb_k_prep, 16) || !aligned(a->cb_v_prep, 16))
      return fail(LOOPVQ_ERR_MISALIGNED, "pool and prepared codebooks must be 16-byte aligned");
  }
  if (cfg->prefix_tokens > 0 && (!a->k_prefix || !a->v_prefix))
    return fail(LOOPVQ_ERR_INVALID_ARG, "prefix windows must not be NULL when prefix_tokens > 0");
  if (cfg->recent_tokens > 0 && (!a->k_recent || !a->v_recent))
    return fail(LOOPVQ_ERR_INVALID_ARG, "recent windows must not be NULL when recent_tokens > 0");
  if ((a->k_prefix && !aligned(a->k_prefix, 16)) || (a->v_prefix && !aligned(a->v_prefix, 16)) ||
      (a->k_recent && !aligned(a->k_recent, 16)) || (a->v_recent && !aligned(a->v_recent, 16)))
    return fail(LOOPVQ_ERR_MISALIGNED, "window buffers must be 16-byte aligned");
  if (!aligned(a->q, 2) || !aligned(a->out, 4) || (a->lse && !aligned(a->lse, 4)) || (a->rot && !aligned(a->rot, 4)) ||
      !aligned(a->seq_lens, 4))
    return fail(LOOPVQ_ERR_MISALIGNED, "q, out, lse, rot or seq_lens misaligned");
  const int S = a->num_splits > 0 ? a->num_splits : plan_splits(cfg, a->batch, a->max_seq_len);
  if (S < min_splits(cfg, a->max_seq_len) || S > 256)
    return fail(LOOPVQ_ERR_INVALID_ARG, "num_splits %d: a context of %d tokens needs between %d and 256 splits", S,
                a->max_seq_len, min_splits(cfg, a->max_seq_len));
  if (can_vq && int64_t(a->max_seq_len) - cfg->prefix_tokens - cfg->recent_tokens >
                    int64_t(a->max_pages_per_seq) * cfg->page_tokens)
    return fail(LOOPVQ_ERR_INVALID_ARG,
                "max_pages_per_seq (%d) pages of %d tokens cannot hold the %lld vector-quantized tokens of "
                "max_seq_len %d", a->max_pages_per_seq, cfg->page_tokens,
                (long long)(int64_t(a->max_seq_len) - cfg->prefix_tokens - cfg->recent_tokens), a->max_seq_len);
  if (can_vq && int64_t(a->num_pages) * z.page_bytes > INT32_MAX)
    return fail(LOOPVQ_ERR_UNSUPPORTED, "num_pages * page_bytes (one kv-head's page region) must stay below 2 GiB");
  const int64_t Q = int64_t(a->batch) * cfg->num_q_heads;
  *need_out = S > 1 ? size_t(S) * Q * (cfg->head_dim + 4) * sizeof(float) : 0;

  const int j = a->loop / cfg->loop_group;
  const int jcb = cfg->codebook_per_loop_group ? j : 0;
  lvq::DecodeParams p{};
  p.B = a->batch;
  p.Hq = cfg->num_q_heads;
  p.Hkv = cfg->num_kv_heads;
  p.d = cfg->head_dim;
  p.P = cfg->prefix_tokens;
  p.R = cfg->recent_tokens;
  p.G = cfg->loop_group;
  p.pt_shift = ilog2(cfg->page_tokens);
  p.max_pages = can_vq ? a->max_pages_per_seq : 0;
  p.max_seq_len = a->max_seq_len;
  p.S = S;
  p.tau = a->loop % cfg->loop_group;
  p.num_pages = a->num_pages;
  p.page_bytes = z.page_bytes;
  p.kind_bytes = z.kind_bytes;
  const float scale = a->softmax_scale > 0.f ? a->softmax_scale : 1.0f / std::sqrt(float(cfg->head_dim));
  p.scale_log2 = scale * 1.4426950408889634f;
  p.q = a->q;
  p.seq_lens = a->seq_lens;
  p.block_table = a->block_table;
  p.head_stride = a->num_pages * z.page_bytes;
  p.pool_lj = can_vq ? a->pool + (int64_t(a->layer) * z.J + j) * cfg->num_kv_heads * p.head_stride : nullptr;
  const int64_t set0 = (int64_t(a->layer) * z.Jcb + jcb) * cfg->num_kv_heads;
  const int64_t set_elems = int64_t(cfg->loop_group) * z.K * cfg->head_dim;
  p.cbk = can_vq ? a->cb_k_prep + set0 * set_elems : nullptr;
  p.cbv = can_vq ? a->cb_v_prep + set0 * set_elems : nullptr;
  p.k_prefix = a->k_prefix;
  p.v_prefix = a->v_prefix;
  p.k_recent = a->k_recent;
  p.v_recent = a->v_recent;
  p.rot = a->rot;
  p.out = a->out;
  p.lse = a->lse;
  p.ws = nullptr;
  *out = p;
  return LOOPVQ_OK;
}

}  // namespace

extern "C" {

loopvq_status loopvq_config_check(const loopvq_config* cfg) {
  const loopvq_status s = check_config(cfg);
  return s == LOOPVQ_OK ? ok() : s;
}

double loopvq_bits_per_elem(const loopvq_config* cfg) {
  if (check_config(cfg) != LOOPVQ_OK) return -1.0;
  return double(cfg->index_bits) / double(cfg->chans_per_group * cfg->loop_group);
}

loopvq_status loopvq_layout_query(const loopvq_config* cfg, int32_t batch, int64_t num_pages, loopvq_layout* out) {
  loopvq_status s = check_config(cfg);
  if (s) return s;
  if (!out) return fail(LOOPVQ_ERR_INVALID_ARG, "out is NULL");
  if (batch < 1) return fail(LOOPVQ_ERR_INVALID_ARG, "batch must be >= 1");
  if (num_pages < 1) return fail(LOOPVQ_ERR_INVALID_ARG, "num_pages must be >= 1");
  const Sizes z = sizes_of(cfg);
  out->tile_bytes = z.tile_bytes;
  out->kind_bytes = z.kind_bytes;
  out->page_bytes = z.page_bytes;
  out->pool_head_stride_bytes = num_pages * z.page_bytes;
  out->pool_bytes = int64_t(cfg->num_layers) * z.J * cfg->num_kv_heads * out->pool_head_stride_bytes;
  out->codebook_elems = int64_t(cfg->num_layers) * z.Jcb * cfg->num_kv_heads * z.ng * z.K * z.E;
  out->norms_elems = int64_t(cfg->num_layers) * z.Jcb * cfg->num_kv_heads * z.ng * z.K;
  out->prefix_elems = int64_t(batch) * cfg->num_kv_heads * cfg->prefix_tokens * cfg->head_dim;
  out->recent_elems = int64_t(batch) * cfg->num_kv_heads * cfg->recent_tokens * cfg->head_dim;
  out->bits_per_elem = double(cfg->index_bits) / double(cfg->chans_per_group * cfg->loop_group);
  return ok();
}

loopvq_status loopvq_codebook_prepare(const loopvq_config* cfg, const uint16_t* cb, uint16_t* cb_prep,
                                      float* cb_norms, void* stream) {
  loopvq_status s = check_config(cfg);
  if (s) return s;
  if (!cb || !cb_prep) return fail(LOOPVQ_ERR_INVALID_ARG, "cb and cb_prep must not be NULL");
  if (!aligned(cb, 16) || !aligned(cb_prep, 16) || (cb_norms && !aligned(cb_norms, 16)))
    return fail(LOOPVQ_ERR_MISALIGNED, "codebook pointers must be 16-byte aligned");
  const Sizes z = sizes_of(cfg);
  lvq::PrepareParams p{};
  p.sets = int64_t(cfg->num_layers) * z.Jcb * cfg->num_kv_heads;
  p.NG = z.ng;
  p.K = z.K;
  p.c = cfg->chans_per_group;
  p.G = cfg->loop_group;
  p.d = cfg->head_dim;
  p.cb = cb;
  p.prep = cb_prep;
  p.norms = cb_norms;
  const hipError_t e = lvq::launch_prepare(p, (hipStream_t)stream);
  if (e != hipSuccess) return fail(LOOPVQ_ERR_HIP, "codebook_prepare launch: %s", hipGetErrorString(e));
  return ok();
}

loopvq_status loopvq_codebook_prepare_groups(const loopvq_config* cfg, const uint16_t* cb, uint16_t* cb_grp,
                                             void* stream) {
  loopvq_status s = check_config(cfg);
  if (s) return s;
  if (!cb || !cb_grp) return fail(LOOPVQ_ERR_INVALID_ARG, "cb and cb_grp must not be NULL");
  if (!aligned(cb, 16) || !aligned(cb_grp, 16)) return fail(LOOPVQ_ERR_MISALIGNED, "codebook pointers must be 16-byte aligned");
  const Sizes z = sizes_of(cfg);
  lvq::PrepareParams p{};
  p.sets = int64_t(cfg->num_layers) * z.Jcb * cfg->num_kv_heads;
  p.NG = z.ng;
  p.K = z.K;
  p.c = cfg->chans_per_group;
  p.G = cfg->loop_group;
  p.d = cfg->head_dim;
  p.cb = cb;
  p.prep = cb_grp;
  const hipError_t e = lvq::launch_prepare_groups(p, (hipStream_t)stream);
  if (e != hipSuccess) return fail(LOOPVQ_ERR_HIP, "codebook_prepare_groups launch: %s", hipGetErrorString(e));
  return ok();
}

loopvq_status loopvq_encode(const loopvq_config* cfg, const loopvq_encode_args* a, void* stream) {
  loopvq_status s = check_config(cfg);
  if (s) return s;
  if (!a) return fail(LOOPVQ_ERR_INVALID_ARG, "args is NULL");
  if ((s = check_supported(cfg))) return s;
  const Sizes z = sizes_of(cfg);
  if (a->layer < 0 || a->layer >= cfg->num_layers) return fail(LOOPVQ_ERR_INVALID_ARG, "layer out of range");
  if (a->loop_group < 0 || a->loop_group >= z.J) return fail(LOOPVQ_ERR_INVALID_ARG, "loop_group out of range");
  if (a->kind != 0 && a->kind != 1) return fail(LOOPVQ_ERR_INVALID_ARG, "kind must be 0 (K) or 1 (V)");
  if (a->n_tokens < 0) return fail(LOOPVQ_ERR_INVALID_ARG, "n_tokens must be >= 0");
  if (a->pool && (a->batch < 1 || a->max_pages_per_seq < 1 || a->num_pages < 1))
    return fail(LOOPVQ_ERR_INVALID_ARG, "batch, max_pages_per_seq and num_pages must be >= 1");
  if (!a->src || !a->cb || !a->cb_norms) return fail(LOOPVQ_ERR_INVALID_ARG, "src, cb and cb_norms must not be NULL");
  if (a->pool && (!a->seq_id || !a->vq_pos || !a->block_table))
    return fail(LOOPVQ_ERR_INVALID_ARG, "seq_id, vq_pos and block_table must not be NULL when pool is given");
  if (!a->pool && !a->out_idx) return fail(LOOPVQ_ERR_INVALID_ARG, "an encode without a pool needs out_idx");
  const int vec = cfg->chans_per_group;  // elements per aligned load (8 B at c=4, 16 B at c=8)
  if (!aligned(a->src, 2 * vec) || a->stride_loop % vec || a->stride_token % vec || a->stride_head % vec)
    return fail(LOOPVQ_ERR_MISALIGNED, "src must be %d-byte aligned and its strides multiples of %d elements",
                2 * vec, vec);
  if (!aligned(a->cb, 16) || !aligned(a->cb_norms, 16))
    return fail(LOOPVQ_ERR_MISALIGNED, "cb and cb_norms must be 16-byte aligned");
  if (a->out_idx && !aligned(a->out_idx, 4)) return fail(LOOPVQ_ERR_MISALIGNED, "out_idx must be 4-byte aligned");
  if (a->rerank_count && !aligned(a->rerank_count, 8))
    return fail(LOOPVQ_ERR_MISALIGNED, "rerank_count must be 8-byte aligned");
  lvq::EncodeParams p = a->pool ? encode_params(cfg, z, a->batch, a->max_pages_per_seq, a->num_pages)
                                : encode_params(cfg, z, 1, 1, 1);
  p.n_slices = 1;
  p.layer = a->layer;
  p.loop_group = a->loop_group;
  p.kind = a->kind;
  p.n_tokens = a->n_tokens;
  p.src = a->src;
  p.stride_loop = a->stride_loop;
  p.stride_token = a->stride_token;
  p.stride_head = a->stride_head;
  p.seq_id = a->seq_id;
  p.vq_pos = a->vq_pos;
  p.block_table = a->block_table;
  // the kernel takes the kind-1 codebook fields for kind 1: an encode's one codebook serves both
  p.cb = p.cb_v = a->cb;
  p.norms = p.norms_v = a->cb_norms;
  p.src_v = a->src;
  p.pool = a->pool;
  p.out_idx = a->out_idx;
  p.rerank_count = a->rerank_count;
  const hipError_t e = lvq::launch_encode(p, cfg->chans_per_group, (hipStream_t)stream);
  if (e != hipSuccess) return fail(LOOPVQ_ERR_HIP, "encode launch: %s", hipGetErrorString(e));
  return ok();
}

loopvq_status loopvq_lloyd_workspace(const loopvq_config* cfg, int32_t n_samples, size_t* bytes) {
  loopvq_status s = check_config(cfg);
  if (s) return s;
  if ((s = check_supported(cfg))) return s;
  if (!bytes) return fail(LOOPVQ_ERR_INVALID_ARG, "bytes is NULL");
  if (n_samples < 0) return fail(LOOPVQ_ERR_INVALID_ARG, "n_samples must be >= 0");
  *bytes = lloyd_plan(cfg, sizes_of(cfg), n_samples).bytes();
  return ok();
}

loopvq_status loopvq_lloyd_update(const loopvq_config* cfg, const loopvq_lloyd_args* a, void* stream) {
  loopvq_status s = check_lloyd(cfg, a);
  if (s) return s;
  const Sizes z = sizes_of(cfg);
  const LloydPlan pl = lloyd_plan(cfg, z, a->n_samples);
  const int64_t set = int64_t(a->layer) * z.Jcb + a->cb_set;
  const int64_t set_codes = int64_t(cfg->num_kv_heads) * z.ng * z.K;
  lvq::LloydParams p{};
  p.n = a->n_samples;
  p.Hkv = cfg->num_kv_heads;
  p.NG = z.ng;
  p.G = cfg->loop_group;
  p.d = cfg->head_dim;
  p.E = z.E;
  p.chunks_a = pl.chunks_a;
  p.rows_a = pl.rows_a;
  p.src = a->src;
  p.stride_loop = a->stride_loop;
  p.stride_token = a->stride_token;
  p.stride_head = a->stride_head;
  p.weight = a->weight;
  p.assign = a->assign;
  p.cb = a->cb + set * set_codes * z.E;
  p.norms = a->cb_norms + set * set_codes;
  p.part_sums = (double*)a->workspace;
  p.part_dist = p.part_sums + pl.sums_doubles;
  p.part_w = p.part_dist + pl.dist_doubles;
  p.cluster_weight = a->cluster_weight;
  p.distortion = a->distortion;
  const hipError_t he = lvq::launch_lloyd(p, cfg->chans_per_group, (hipStream_t)stream);
  if (he != hipSuccess) return fail(LOOPVQ_ERR_HIP, "lloyd update launch: %s", hipGetErrorString(he));
  return ok();
}

loopvq_status loopvq_lloyd_step(const loopvq_config* cfg, const loopvq_lloyd_args* a, void* stream) {
  loopvq_status s = check_lloyd(cfg, a);
  if (s) return s;
  if (a->n_samples > 0) {   // the assignment: the encode kernels, without a pool
    const Sizes z = sizes_of(cfg);
    lvq::EncodeParams e = encode_params(cfg, z, 1, 1, 1);
    e.n_slices = 1;
    e.layer = a->layer;
    e.loop_group = a->cb_set;   // selects the codebook set; with no pool nothing else reads it
    e.kind = 0;
    e.n_tokens = a->n_samples;
    e.src = e.src_v = a->src;
    e.stride_loop = a->stride_loop;
    e.stride_token = a->stride_token;
    e.stride_head = a->stride_head;
    e.cb = e.cb_v = a->cb;
    e.norms = e.norms_v = a->cb_norms;
    e.pool = nullptr;
    e.out_idx = a->assign;
    e.rerank_count = a->rerank_count;
    const hipError_t he = lvq::launch_encode(e, cfg->chans_per_group, (hipStream_t)stream);
    if (he != hipSuccess) return fail(LOOPVQ_ERR_HIP, "lloyd assignment launch: %s", hipGetErrorString(he));
  }
  return loopvq_lloyd_update(cfg, a, stream);
}

loopvq_status loopvq_evict(const loopvq_config* cfg, const loopvq_evict_args* a, void* stream) {
  loopvq_status s = check_config(cfg);
  if (s) return s;
  if (!a) return fail(LOOPVQ_ERR_INVALID_ARG, "args is NULL");
  if ((s = check_supported(cfg))) return s;
  const Sizes z = sizes_of(cfg);
  if (cfg->recent_tokens < 1) return fail(LOOPVQ_ERR_INVALID_ARG, "eviction needs recent_tokens >= 1");
  if (a->batch < 1 || a->max_pages_per_seq < 1 || a->num_pages < 1)
    return fail(LOOPVQ_ERR_INVALID_ARG, "batch, max_pages_per_seq and num_pages must be >= 1");
  if (!a->k_ring || !a->v_ring || !a->ring_slot || !a->vq_pos || !a->block_table || !a->cb_k || !a->cb_v ||
      !a->norms_k || !a->norms_v || !a->pool)
    return fail(LOOPVQ_ERR_INVALID_ARG,
                "k_ring, v_ring, ring_slot, vq_pos, block_table, cb_k, cb_v, norms_k, norms_v and pool must not be "
                "NULL");
  if (!aligned(a->k_ring, 16) || !aligned(a->v_ring, 16))
    return fail(LOOPVQ_ERR_MISALIGNED, "k_ring and v_ring must be 16-byte aligned");
  if (!aligned(a->cb_k, 16) || !aligned(a->cb_v, 16) || !aligned(a->norms_k, 16) || !aligned(a->norms_v, 16))
    return fail(LOOPVQ_ERR_MISALIGNED, "codebooks and norms must be 16-byte aligned");
  if (a->out_idx && !aligned(a->out_idx, 4)) return fail(LOOPVQ_ERR_MISALIGNED, "out_idx must be 4-byte aligned");
  if (a->rerank_count && !aligned(a->rerank_count, 8))
    return fail(LOOPVQ_ERR_MISALIGNED, "rerank_count must be 8-byte aligned");
  if (int64_t(cfg->num_layers) * z.J * 2 * cfg->num_kv_heads * (z.ng / 4) > (int64_t(1) << 31) - 1)
    return fail(LOOPVQ_ERR_INVALID_ARG, "too many slices for one launch");
  const int64_t R = cfg->recent_tokens, d = cfg->head_dim;
  lvq::EncodeParams p = encode_params(cfg, z, a->batch, a->max_pages_per_seq, a->num_pages);
  p.n_slices = cfg->num_layers * z.J * 2;
  p.n_tokens = a->batch;
  p.R = cfg->recent_tokens;
  p.src = a->k_ring;
  p.src_v = a->v_ring;
  p.stride_head = R * d;
  p.stride_token = cfg->num_kv_heads * R * d;          // sequence b
  p.stride_loop = int64_t(a->batch) * p.stride_token;   // loop step t
  p.stride_slot = d;
  p.seq_id = nullptr;
  p.vq_pos = a->vq_pos;
  p.row_slot = a->ring_slot;
  p.block_table = a->block_table;
  p.cb = a->cb_k;
  p.cb_v = a->cb_v;
  p.norms = a->norms_k;
  p.norms_v = a->norms_v;
  p.pool = a->pool;
  p.out_idx = a->out_idx;
  p.rerank_count = a->rerank_count;
  const hipError_t e = lvq::launch_encode(p, cfg->chans_per_group, (hipStream_t)stream);
  if (e != hipSuccess) return fail(LOOPVQ_ERR_HIP, "evict launch: %s", hipGetErrorString(e));
  return ok();
}

loopvq_status loopvq_decode_attn_workspace(const loopvq_config* cfg, int32_t batch, int32_t max_seq_len,
                                           size_t* bytes) {
  loopvq_status s = check_config(cfg);
  if (s) return s;
  if (!bytes) return fail(LOOPVQ_ERR_INVALID_ARG, "bytes is NULL");
  if (batch < 1 || max_seq_len < 1) return fail(LOOPVQ_ERR_INVALID_ARG, "batch and max_seq_len must be >= 1");
  const int S = plan_splits(cfg, batch, max_seq_len);
  *bytes = S > 1 ? size_t(S) * batch * cfg->num_q_heads * (cfg->head_dim + 4) * sizeof(float) : 0;
  return ok();
}

loopvq_status loopvq_decode_attn(const loopvq_config* cfg, const loopvq_decode_args* a, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  lvq::DecodeParams p;
  size_t need = 0;
  const loopvq_status s = decode_setup(cfg, a, &p, &need);
  if (s) return s;
  if (workspace_bytes < need || (need && !workspace))
    return fail(LOOPVQ_ERR_WORKSPACE, "workspace too small: %zu bytes needed for %d splits", need, p.S);
  if (need && !aligned(workspace, 16)) return fail(LOOPVQ_ERR_MISALIGNED, "workspace must be 16-byte aligned");
  p.ws = static_cast<float*>(workspace);
  const hipError_t e = lvq::launch_decode(p, cfg->head_dim / cfg->chans_per_group, cfg->chans_per_group,
                                          (hipStream_t)stream);
  if (e != hipSuccess) return fail(LOOPVQ_ERR_HIP, "decode_attn launch: %s", hipGetErrorString(e));
  return ok();
}

loopvq_status loopvq_decode_attn_noalloc(const loopvq_config* cfg, const loopvq_decode_args* a, void* stream) {
  lvq::DecodeParams p;
  size_t need = 0;
  const loopvq_status s = decode_setup(cfg, a, &p, &need);
  if (s) return s;
  if (need > lvq::kDecodeStaticScratchBytes)
    return fail(LOOPVQ_ERR_WORKSPACE,
                "the split plan (%d splits) needs %zu bytes of partials; the static scratch holds %zu bytes", p.S,
                need, lvq::kDecodeStaticScratchBytes);
  if (need) {
    void* ws = nullptr;
    const hipError_t e = lvq::decode_static_scratch(&ws);
    if (e != hipSuccess) return fail(LOOPVQ_ERR_HIP, "static decode scratch lookup: %s", hipGetErrorString(e));
    p.ws = static_cast<float*>(ws);
  }
  const hipError_t e = lvq::launch_decode(p, cfg->head_dim / cfg->chans_per_group, cfg->chans_per_group,
                                          (hipStream_t)stream);
  if (e != hipSuccess) return fail(LOOPVQ_ERR_HIP, "decode_attn_noalloc launch: %s", hipGetErrorString(e));
  return ok();
}

loopvq_status loopvq_extend_attn(const loopvq_config* cfg, const loopvq_extend_args* a, void* stream) {
  loopvq_status s = check_config(cfg);
  if (s) return s;
  if (!a) return fail(LOOPVQ_ERR_INVALID_ARG, "args is NULL");
  if ((s = check_supported(cfg))) return s;
  const Sizes z = sizes_of(cfg);
  if (a->layer < 0 || a->layer >= cfg->num_layers) return fail(LOOPVQ_ERR_INVALID_ARG, "layer out of range");
  if (a->loop < 0 || a->loop >= cfg->num_loops) return fail(LOOPVQ_ERR_INVALID_ARG, "loop out of range");
  if (a->batch < 1 || a->chunk < 1) return fail(LOOPVQ_ERR_INVALID_ARG, "batch and chunk must be >= 1");
  if (a->max_seq_len < 0) return fail(LOOPVQ_ERR_INVALID_ARG, "max_seq_len must be >= 0");
  const int grp = cfg->num_q_heads / cfg->num_kv_heads;
  const int rows_wg = 256;   // query rows per workgroup of the kernel
  const int64_t row_blocks = (int64_t(a->chunk) * grp + rows_wg - 1) / rows_wg;
  if (int64_t(a->batch) * cfg->num_kv_heads * row_blocks > (int64_t(1) << 31) - 1)
    return fail(LOOPVQ_ERR_INVALID_ARG, "batch * kv_heads * chunk too large for one launch");
  if (!a->q || !a->k_new || !a->v_new || !a->seq_lens || !a->out)
    return fail(LOOPVQ_ERR_INVALID_ARG, "q, k_new, v_new, seq_lens and out must not be NULL");
  const bool can_vq = int64_t(a->max_seq_len) > int64_t(cfg->prefix_tokens) + cfg->recent_tokens;
  if (can_vq) {
    if (!a->block_table || !a->pool || !a->cb_k_grp || !a->cb_v_grp)
      return fail(LOOPVQ_ERR_INVALID_ARG, "block_table, pool and group-major codebooks must not be NULL");
    if (a->max_pages_per_seq < 1 || a->num_pages < 1)
      return fail(LOOPVQ_ERR_INVALID_ARG, "max_pages_per_seq and num_pages must be >= 1");
    if (int64_t(a->max_pages_per_seq) * cfg->page_tokens > INT32_MAX)
      return fail(LOOPVQ_ERR_INVALID_ARG, "max_pages_per_seq * page_tokens must stay below 2^31");
    if (int64_t(a->max_seq_len) - cfg->prefix_tokens - cfg->recent_tokens >
        int64_t(a->max_pages_per_seq) * cfg->page_tokens)
      return fail(LOOPVQ_ERR_INVALID_ARG,
                  "max_pages_per_seq (%d) pages of %d tokens cannot hold the %lld vector-quantized tokens of "
                  "max_seq_len %d", a->max_pages_per_seq, cfg->page_tokens,
                  (long long)(int64_t(a->max_seq_len) - cfg->prefix_tokens - cfg->recent_tokens), a->max_seq_len);
    if (!aligned(a->pool, 16) || !aligned(a->cb_k_grp, 16) || !aligned(a->cb_v_grp, 16))
      return fail(LOOPVQ_ERR_MISALIGNED, "pool and group-major codebooks must be 16-byte aligned");
  }
  if (cfg->prefix_tokens > 0 && (!a->k_prefix || !a->v_prefix))
    return fail(LOOPVQ_ERR_INVALID_ARG, "prefix windows must not be NULL when prefix_tokens > 0");
  if (cfg->recent_tokens > 0 && (!a->k_recent || !a->v_recent))
    return fail(LOOPVQ_ERR_INVALID_ARG, "recent windows must not be NULL when recent_tokens > 0");
  if ((a->k_prefix && !aligned(a->k_prefix, 16)) || (a->v_prefix && !aligned(a->v_prefix, 16)) ||
      (a->k_recent && !aligned(a->k_recent, 16)) || (a->v_recent && !aligned(a->v_recent, 16)) ||
      !aligned(a->k_new, 16) || !aligned(a->v_new, 16) || !aligned(a->q, 16))
    return fail(LOOPVQ_ERR_MISALIGNED, "q, chunk and window buffers must be 16-byte aligned");
  if (!aligned(a->out, 16) || (a->rot && !aligned(a->rot, 4)) || !aligned(a->seq_lens, 4) ||
      (a->chunk_lens && !aligned(a->chunk_lens, 4)) || (a->lse && !aligned(a->lse, 4)))
    return fail(LOOPVQ_ERR_MISALIGNED, "out (16 bytes), rot, seq_lens, chunk_lens or lse misaligned");

  const int j = a->loop / cfg->loop_group;
  const int jcb = cfg->codebook_per_loop_group ? j : 0;
  lvq::ExtendParams p{};
  p.B = a->batch;
  p.Hq = cfg->num_q_heads;
  p.Hkv = cfg->num_kv_heads;
  p.P = cfg->prefix_tokens;
  p.R = cfg->recent_tokens;
  p.G = cfg->loop_group;
  p.M = a->chunk;
  p.row_blocks = (int)row_blocks;
  p.pt_shift = ilog2(cfg->page_tokens);
  p.max_pages = can_vq ? a->max_pages_per_seq : 0;
  p.max_seq_len = a->max_seq_len;
  p.tau = a->loop % cfg->loop_group;
  p.num_pages = a->num_pages;
  p.page_bytes = z.page_bytes;
  p.kind_bytes = z.kind_bytes;
  p.head_stride = a->num_pages * z.page_bytes;
  const float scale = a->softmax_scale > 0.f ? a->softmax_scale : 1.0f / std::sqrt(float(cfg->head_dim));
  p.scale_log2 = scale * 1.4426950408889634f;
  p.q = a->q;
  p.k_new = a->k_new;
  p.v_new = a->v_new;
  p.seq_lens = a->seq_lens;
  p.chunk_lens = a->chunk_lens;
  p.block_table = a->block_table;
  p.pool_lj = can_vq ? a->pool + (int64_t(a->layer) * z.J + j) * cfg->num_kv_heads * p.head_stride : nullptr;
  const int64_t set0 = (int64_t(a->layer) * z.Jcb + jcb) * cfg->num_kv_heads;
  const int64_t set_elems = int64_t(cfg->loop_group) * z.K * cfg->head_dim;
  p.cbk = can_vq ? a->cb_k_grp + set0 * set_elems : nullptr;
  p.cbv = can_vq ? a->cb_v_grp + set0 * set_elems : nullptr;
  p.k_prefix = a->k_prefix;
  p.v_prefix = a->v_prefix;
  p.k_recent = a->k_recent;
  p.v_recent = a->v_recent;
  p.rot = a->rot;
  p.out = a->out;
  p.lse = a->lse;
  const hipError_t e = lvq::launch_extend(p, z.ng, cfg->chans_per_group, (hipStream_t)stream);
  if (e != hipSuccess) return fail(LOOPVQ_ERR_HIP, "extend_attn launch: %s", hipGetErrorString(e));
  return ok();
}

const char* loopvq_status_string(loopvq_status s) {
  switch (s) {
    case LOOPVQ_OK: return "ok";
    case LOOPVQ_ERR_INVALID_ARG: return "invalid argument";
    case LOOPVQ_ERR_UNSUPPORTED: return "unsupported variant";
    case LOOPVQ_ERR_MISALIGNED: return "misaligned pointer";
    case LOOPVQ_ERR_WORKSPACE: return "workspace too small";
    case LOOPVQ_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* loopvq_last_error(void) { return g_err; }

}  // extern "C"
