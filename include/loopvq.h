/*
 * loopvq.h - C ABI of the LoopVQ decode-attention / encode library (MI355X, gfx950).
 *
 * LoopVQ ("LoopVQ: Sub 1-bit KV Cache Quantization for Looped Transformers",
 * arXiv 2611.05304; English abstract on the shd-paper.top listing) stores the
 * per-loop-step KV cache of a looped transformer as codebook indices: one
 * b-bit index covers c channels of G consecutive loop steps (airadar.tv
 * summary, opening paragraph), i.e. b / (c*G) bits per element (0.5 at
 * c=4, G=4, b=8; 0.25 at c=8).  The first P prefix and last R recent tokens
 * of every sequence stay bf16 (airadar.tv summary, section "Utilisation").
 * The serving path stores the indices packed and decodes with fused kernels
 * (airadar.tv summary, section "Raisons"); this library is that path.
 *
 * Conventions for every entry point
 *   - All sizes are element counts unless a name ends in _bytes.
 *   - bf16 tensors are passed as uint16_t bit patterns.
 *   - Device pointers are HIP device addresses of memory the CALLER owns; the
 *     library never allocates, frees or synchronises, and keeps no state other
 *     than a thread-local error string.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream).  Launches are
 *     asynchronous; faults inside a kernel surface at the caller's next
 *     synchronisation on that stream.
 *   - Every host-detectable problem (bad configuration, NULL or misaligned
 *     pointer, unsupported variant, small workspace) returns a negative status
 *     BEFORE any HIP call, with no partial work; loopvq_last_error() then holds a
 *     description.  A failed launch returns LOOPVQ_ERR_HIP.
 *   - Calls are reentrant; two calls that write the same buffers race.
 */
#ifndef LOOPVQ_H
#define LOOPVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t loopvq_status;
#define LOOPVQ_OK 0
#define LOOPVQ_ERR_INVALID_ARG (-1)
#define LOOPVQ_ERR_UNSUPPORTED (-2)
#define LOOPVQ_ERR_MISALIGNED (-3)
#define LOOPVQ_ERR_WORKSPACE (-4)
#define LOOPVQ_ERR_HIP (-5)

/* Model / cache shape.  All fields int32.
 *   num_layers L, num_loops T, loop_group G (T % G == 0: a loop group is the
 *   G consecutive loop steps [j*G, j*G+G) sharing one index, J = T/G groups);
 *   num_q_heads Hq, num_kv_heads Hkv (Hq % Hkv == 0), head_dim d,
 *   chans_per_group c (d % c == 0, NG = d/c channel groups, NG % 4 == 0),
 *   index_bits b in [1,16] (K = 2^b codewords), prefix_tokens P and
 *   recent_tokens R (bf16 windows), page_tokens PT (tokens per index page, a
 *   power of two >= 64), codebook_per_loop_group (0: one codebook set per
 *   (layer, kv-head, group) shared by all loop groups, Jcb = 1; 1: one per loop
 *   group, Jcb = J).
 * Kernels are built for b = 8, (c, G) in {(4,4), (8,4), (8,2), (4,8)} (sub-vectors
 * of 16 or 32 elements) and (c, d) in {(4,64), (4,128), (8,128)}; other valid
 * shapes return LOOPVQ_ERR_UNSUPPORTED from the compute entry points.  A model
 * that picks (c, G) per layer or per loop group uses one config (and one pool
 * and codebook set) per distinct choice. */
typedef struct loopvq_config {
  int32_t num_layers;
  int32_t num_loops;
  int32_t loop_group;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t chans_per_group;
  int32_t index_bits;
  int32_t prefix_tokens;
  int32_t recent_tokens;
  int32_t page_tokens;
  int32_t codebook_per_loop_group;
} loopvq_config;

/* Byte sizes and strides of every buffer the library reads or writes.
 *
 * Index pool (uint8): [L][J][Hkv][num_pages][page_bytes].  A page holds the
 * packed indices of PT consecutive vector-quantized positions of one
 * (layer, loop group, kv-head): [kind: K then V][PT/4 token quads][NG/4 group
 * quads][micro-tile of 2*b bytes].  A micro-tile packs 16 indices: element
 * e = 4*i + r is token 4*Q + i, group 4*u + r; bit beta of element e sits at
 * bit e*b + beta of the tile read as a little-endian integer.  Unwritten
 * slots must be zero (zero the pool before the first encode).
 * A block table int32 [B][max_pages_per_seq] maps (sequence, vq_position/PT)
 * to a page index; vq_position u of token n is n - P.
 *
 * Canonical codebooks (bf16): [L][Jcb][Hkv][NG][K][c*G]; row k of group g is a
 * sub-vector in loop-major order (element tau*c + i = channel g*c + i of loop
 * step tau of the group).  K and V have separate codebooks.
 * Prepared codebooks (bf16, written by loopvq_codebook_prepare):
 * [L][Jcb][Hkv][G][K][d], so the loop-step-tau slice of a codebook set is one
 * contiguous K x d block; norms (fp32): [L][Jcb][Hkv][NG][K] squared norms.
 * Windows (bf16) for one (layer, loop step): prefix [B][Hkv][P][d], recent
 * [B][Hkv][R][d]; rows [0, n_prefix) and [0, n_recent) are read. */
typedef struct loopvq_layout {
  int64_t tile_bytes;
  int64_t kind_bytes;
  int64_t page_bytes;
  int64_t pool_head_stride_bytes; /* num_pages * page_bytes */
  int64_t pool_bytes;             /* L * J * Hkv * num_pages * page_bytes */
  int64_t codebook_elems;         /* bf16 elements of one canonical (or prepared) codebook set, K or V */
  int64_t norms_elems;            /* fp32 elements of one norms array */
  int64_t prefix_elems;           /* bf16 elements of one prefix window buffer, for one (l, t) */
  int64_t recent_elems;           /* bf16 elements of one recent window buffer, for one (l, t) */
  double bits_per_elem;           /* b / (c*G) */
} loopvq_layout;

/* Validate a configuration: the rules above (ranges, divisibility, page size).
 * Source: one codebook index covers c channels of G consecutive loop steps
 * (airadar.tv summary, opening paragraph; arXiv 2611.05304 English abstract:
 * the channels of several loop steps are coded jointly), so T must split into
 * whole loop groups and d into whole channel groups; P and R are the bf16
 * prefix / recent token counts of the serving launch line (airadar.tv summary,
 * section "Utilisation": 8 and 64).
 * Returns LOOPVQ_OK or LOOPVQ_ERR_INVALID_ARG; never touches the GPU. */
loopvq_status loopvq_config_check(const loopvq_config* cfg);

/* Index bits per cache element, b / (c*G) (0.5 and 0.25 are the operating
 * points in the arXiv 2611.05304 abstract).  Returns -1.0 for an invalid config. */
double loopvq_bits_per_elem(const loopvq_config* cfg);

/* Fill *out with the sizes above for `batch` sequences and a pool of
 * `num_pages` pages per (layer, loop group, kv-head).  Source: the serving
 * path stores the codebook indices packed (airadar.tv summary, section
 * "Raisons"); the page and micro-tile order above is this library's own
 * reading of that storage, and the bf16 window sizes follow the prefix /
 * recent counts (section "Utilisation").  Host only; returns
 * LOOPVQ_ERR_INVALID_ARG for an invalid config, a NULL out, batch < 1 or
 * num_pages < 1. */
loopvq_status loopvq_layout_query(const loopvq_config* cfg, int32_t batch, int64_t num_pages,
                                  loopvq_layout* out);

/* Derive the decode-side codebook copies from canonical codebooks.
 * Source: the model ships a codebook folder (airadar.tv summary, section
 * "Utilisation") with one codebook per (layer, kv-head, channel group) whose
 * rows span G loop steps (opening paragraph); a decode launch of loop step t
 * only needs slice tau = t mod G of every row, so this copy makes that slice
 * one contiguous block.  Errors: INVALID_ARG (bad config, NULL cb or
 * cb_prep), MISALIGNED, HIP (failed launch).
 *   cb        device, bf16 canonical [L][Jcb][Hkv][NG][K][c*G] (one kind)
 *   cb_prep   device, bf16 prepared  [L][Jcb][Hkv][G][K][d]   (written)
 *   cb_norms  device, fp32 [L][Jcb][Hkv][NG][K] squared norms (written; may be NULL)
 * Pointers 16-byte aligned.  Run once per codebook set, off the per-token path. */
loopvq_status loopvq_codebook_prepare(const loopvq_config* cfg, const uint16_t* cb,
                                      uint16_t* cb_prep, float* cb_norms, void* stream);

/* Group-major loop slices for extend attention: the same codewords as cb, as
 *   cb_grp  device bf16 [L][Jcb][Hkv][G][NG][K][c]  (written),
 * so that the c channels of group g, loop slice tau of every codeword are one
 * contiguous K x c block.  Pointers 16-byte aligned.  Run once per codebook
 * set, like loopvq_codebook_prepare. */
loopvq_status loopvq_codebook_prepare_groups(const loopvq_config* cfg, const uint16_t* cb,
                                             uint16_t* cb_grp, void* stream);

/* Encode: nearest codeword (plain squared Euclidean distance, lowest index on
 * ties) of every sub-vector of n_tokens token rows, for every kv-head and
 * channel group of one (layer, loop group, kind), packed into the pool.
 * Source: a sub-vector groups the channels of G consecutive loop steps and
 * shares one codebook index (airadar.tv summary, opening paragraph; arXiv
 * 2611.05304 English abstract); the indices are stored packed (airadar.tv
 * summary, section "Raisons").  The pages name no distance or tie rule: the
 * squared Euclidean distance and the lowest index are this library's reading.
 * Errors: INVALID_ARG (config, layer / loop group / kind out of range,
 * n_tokens < 0, a NULL pointer the call needs, batch / pages < 1 with a pool),
 * MISALIGNED, UNSUPPORTED (b != 8 or an unbuilt (c, G, d)), HIP (failed
 * launch); n_tokens == 0 returns OK with no launch.
 * Sub-vector (row r, head h, group g) element tau*c + i is
 *   src[tau*stride_loop + r*stride_token + h*stride_head + g*c + i],  tau < G.
 * Distances are screened on bf16 matrix cores in fp32; whenever the two best
 * screened distances are within the screen's rounding bound, every codeword is
 * re-scored exactly in fp64, so the result equals a brute-force fp64 search. */
typedef struct loopvq_encode_args {
  int32_t layer;                /* l in [0, L) */
  int32_t loop_group;           /* j in [0, J) */
  int32_t kind;                 /* 0 = keys, 1 = values */
  int32_t n_tokens;             /* rows to encode (>= 0) */
  const uint16_t* src;          /* device bf16; 16-byte aligned; rows 16-byte aligned */
  int64_t stride_loop;          /* elements between loop steps tau and tau+1 */
  int64_t stride_token;         /* elements between rows r and r+1 */
  int64_t stride_head;          /* elements between kv-heads */
  const int32_t* seq_id;        /* device [n_tokens]: sequence of each row, in [0, batch) */
  const int32_t* vq_pos;        /* device [n_tokens]: vq position u of each row, u >= 0 */
  const int32_t* block_table;   /* device [batch][max_pages_per_seq] */
  int32_t batch;
  int32_t max_pages_per_seq;
  int64_t num_pages;            /* pages per (layer, loop group, kv-head) in the pool */
  const uint16_t* cb;           /* device canonical codebooks of this kind, bf16 */
  const float* cb_norms;        /* device squared norms of this kind (loopvq_codebook_prepare) */
  uint8_t* pool;                /* device index pool (written), or NULL for the assignment alone:
                                   then seq_id, vq_pos, block_table, batch, max_pages_per_seq and
                                   num_pages are not read and out_idx is required */
  int32_t* out_idx;             /* optional device [n_tokens][Hkv][NG] copy of the chosen indices */
  unsigned long long* rerank_count; /* optional device counter: += sub-vectors re-scored in fp64 */
} loopvq_encode_args;

loopvq_status loopvq_encode(const loopvq_config* cfg, const loopvq_encode_args* args, void* stream);

/* Evict: when a new token enters the bf16 recent window of R tokens (airadar.tv
 * summary, section "Utilisation"), the oldest one leaves it and is vector-
 * quantized.  One call encodes that token for every layer, loop group, kind
 * (K and V), kv-head and channel group, exactly as loopvq_encode would, in a
 * single launch (the same screen and exact re-rank).
 * The recent windows are rings: k_ring / v_ring hold bf16
 *   [L][T][B][Hkv][R][d]   (the per-(layer, loop step) window of decode is
 *                           k_ring + (l*T + t) * B*Hkv*R*d),
 * and the leaving token of sequence b is in slot ring_slot[b] of every
 * (layer, loop step, kv-head) ring.  Its indices are written at vq position
 * vq_pos[b] of sequence b in the pool.  A sequence is skipped when
 * vq_pos[b] < 0 or ring_slot[b] is outside [0, R).  After the call returns (on
 * the stream) the caller may overwrite the slot with the incoming token. */
typedef struct loopvq_evict_args {
  int32_t batch;                /* B: sequences (rows of ring_slot, vq_pos, block_table) */
  int32_t max_pages_per_seq;
  int64_t num_pages;            /* pages per (layer, loop group, kv-head) in the pool */
  const uint16_t* k_ring;       /* device bf16 [L][T][B][Hkv][R][d], 16-byte aligned */
  const uint16_t* v_ring;       /* device bf16, same layout */
  const int32_t* ring_slot;     /* device [B] */
  const int32_t* vq_pos;        /* device [B] */
  const int32_t* block_table;   /* device [B][max_pages_per_seq] */
  const uint16_t* cb_k;         /* device canonical key codebooks */
  const uint16_t* cb_v;         /* device canonical value codebooks */
  const float* norms_k;         /* device squared norms of the key codebooks */
  const float* norms_v;
  uint8_t* pool;                /* device index pool (written) */
  int32_t* out_idx;             /* optional device [L][J][2][B][Hkv][NG] copy of the chosen indices */
  unsigned long long* rerank_count; /* optional device counter: += sub-vectors re-scored in fp64 */
} loopvq_evict_args;

loopvq_status loopvq_evict(const loopvq_config* cfg, const loopvq_evict_args* args, void* stream);

/* Lloyd step: one iteration of the weighted k-means that learns the codebooks
 * (airadar.tv summary, opening summary: the codebooks come from k-means weighted
 * by Fisher information).  For the codebook set (layer, cb_set) of one kind
 * (cb_set = loop group j with codebook_per_loop_group, else 0), every kv-head h
 * and channel group g:
 *   1. assignment: a[r][h][g] = nearest codeword of sample r's sub-vector under
 *      the current codebook, lowest index on ties, exactly as loopvq_encode picks
 *      it (the sub-vector of row r is built from the G sample planes like an
 *      encode row: element tau*c + i is channel g*c + i of plane tau);
 *   2. update: codeword k becomes sum_r w[r][h][g] x_r / sum_r w[r][h][g] over the
 *      samples assigned to it, rounded to the nearest bf16 (ties to even); a
 *      codeword whose samples weigh nothing keeps its value.  The sums are fp64
 *      in an unspecified order, so a mean within about 1e-12 (relative) of a
 *      bf16 rounding midpoint may round either way;
 *   3. the set's squared norms in cb_norms are recomputed as
 *      loopvq_codebook_prepare computes them.  The decode-side prepared copy is
 *      not touched: call loopvq_codebook_prepare after the last iteration.
 * Samples: plane tau of row r, kv-head h at src + tau*stride_loop +
 * r*stride_token + h*stride_head (elements), channels contiguous.  The weights
 * stand in for the Fisher information: one per sample and group, finite and
 * >= 0.  All of one call's work is on `stream`; nothing is allocated: the
 * caller passes a workspace of at least loopvq_lloyd_workspace() bytes, which
 * must not be shared by calls that may overlap. */
typedef struct loopvq_lloyd_args {
  int32_t layer;                /* l in [0, L) */
  int32_t cb_set;               /* in [0, Jcb): the loop group with per-group codebooks, else 0 */
  int32_t n_samples;            /* n >= 0 */
  const uint16_t* src;          /* device bf16, 16-byte aligned */
  int64_t stride_loop;          /* elements; all three multiples of 8 */
  int64_t stride_token;
  int64_t stride_head;
  const float* weight;          /* device fp32 [n][Hkv][NG], 16-byte aligned */
  uint16_t* cb;                 /* device canonical codebooks of one kind [L][Jcb][Hkv][NG][K][E]:
                                   the set's codewords are updated in place */
  float* cb_norms;              /* device squared norms of the same kind: the set's are rewritten */
  int32_t* assign;              /* device [n][Hkv][NG], 16-byte aligned: written with step 1
                                   (read by loopvq_lloyd_update) */
  double* cluster_weight;       /* optional device [Hkv][NG][K]: total weight of each codeword */
  double* distortion;           /* optional device [Hkv][NG]: sum_r w ||x_r - C[a_r]||^2 under the
                                   codebook before the update */
  void* workspace;              /* device, 16-byte aligned */
  size_t workspace_bytes;
  unsigned long long* rerank_count; /* optional device counter, as for loopvq_encode */
} loopvq_lloyd_args;

/* Workspace bytes loopvq_lloyd_step and loopvq_lloyd_update need for n_samples samples. */
loopvq_status loopvq_lloyd_workspace(const loopvq_config* cfg, int32_t n_samples, size_t* bytes);

/* Steps 1-3 above. */
loopvq_status loopvq_lloyd_step(const loopvq_config* cfg, const loopvq_lloyd_args* args, void* stream);

/* Steps 2-3 alone, with `assign` an input: the assignment of the same samples
 * under the set's current codebook, e.g. loopvq_encode's out_idx (without a
 * pool).  Same arguments and rules as loopvq_lloyd_step; rerank_count unused. */
loopvq_status loopvq_lloyd_update(const loopvq_config* cfg, const loopvq_lloyd_args* args, void* stream);

/* Decode attention for one (layer l, loop step t) over all B sequences and Hq
 * query heads.  Source: the serving path decodes with fused kernels over the
 * packed indices (airadar.tv summary, section "Raisons"), the first 8 and last
 * 64 tokens stay bf16 (section "Utilisation"), and each loop step reads its
 * own cache (arXiv 2611.05304 English abstract), so a launch reads loop slice
 * t mod G of the codebooks and index group t / G.  For query (b, hq) with
 * kv-head h = hq / (Hq/Hkv) and N =
 * seq_lens[b] cached tokens (the token being decoded included), the keys and
 * values are [prefix rows | vector-quantized rows | recent rows] with
 * n_prefix = min(P, N), n_vq = max(0, N - P - R), n_recent = N - n_prefix - n_vq;
 * a VQ row's channels [g*c, g*c+c) are the loop-step-(t mod G) slice of
 * codeword idx[g] of the (l, t/G) pages.  Output
 *   out[b][hq][:] = sum_n softmax_n(scale * q'.k_n) v_n  (fp32),
 *   lse[b][hq]    = ln sum_n exp(scale * q'.k_n),
 * with q' = R^T q when `rot` (fp32 [d][d] row-major, R[i][j]) is given, else q.
 * The kernel builds a q.codeword lookup table per channel group in LDS, reads
 * the packed indices once, and accumulates V as codeword-index histograms.
 * Tokens are split across workgroups (num_splits, 0 = automatic); splits are
 * merged with log-sum-exp in a second kernel using `workspace`. */
typedef struct loopvq_decode_args {
  int32_t layer;                /* l in [0, L) */
  int32_t loop;                 /* t in [0, T) */
  int32_t batch;                /* B > 0 */
  int32_t max_pages_per_seq;    /* with VQ rows, max_pages_per_seq * PT >= max_seq_len - P - R and
                                   max_pages_per_seq * PT < 2^31 (else LOOPVQ_ERR_INVALID_ARG) */
  int32_t max_seq_len;          /* upper bound of seq_lens[] (sizes the split plan) */
  int32_t num_splits;           /* 0 = automatic, else 1..256 (at least the number a context of
                                   max_seq_len needs: one split holds at most 65,536 VQ rows) */
  int64_t num_pages;            /* pages per (layer, loop group, kv-head); with VQ rows,
                                   num_pages * page_bytes < 2^31 (else LOOPVQ_ERR_UNSUPPORTED) */
  const uint16_t* q;            /* device bf16 [B][Hq][d] */
  const int32_t* seq_lens;      /* device [B], each in [0, max_seq_len].  0 is an empty context:
                                   out row 0, lse -inf.  A length outside [0, max_seq_len] (which
                                   the host cannot see) yields a NaN out row and lse. */
  const int32_t* block_table;   /* device [B][max_pages_per_seq] */
  const uint8_t* pool;          /* device index pool */
  const uint16_t* cb_k_prep;    /* device prepared key codebooks */
  const uint16_t* cb_v_prep;    /* device prepared value codebooks */
  const uint16_t* k_prefix;     /* device bf16 [B][Hkv][P][d] for (l, t); NULL allowed iff P == 0 */
  const uint16_t* v_prefix;
  const uint16_t* k_recent;     /* device bf16 [B][Hkv][R][d] for (l, t); NULL allowed iff R == 0 */
  const uint16_t* v_recent;
  const float* rot;             /* device fp32 [d][d] or NULL */
  float softmax_scale;          /* <= 0 selects 1/sqrt(d) */
  float* out;                   /* device fp32 [B][Hq][d] (written) */
  float* lse;                   /* device fp32 [B][Hq] or NULL */
} loopvq_decode_args;

/* Workspace bytes loopvq_decode_attn needs for this batch and maximum length
 * (the automatic split plan; explicit num_splits needs <= 256 * B*Hq*(d+4)*4). */
loopvq_status loopvq_decode_attn_workspace(const loopvq_config* cfg, int32_t batch,
                                           int32_t max_seq_len, size_t* bytes);

loopvq_status loopvq_decode_attn(const loopvq_config* cfg, const loopvq_decode_args* args,
                                 void* workspace, size_t workspace_bytes, void* stream);

/* loopvq_decode_attn without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, serving loops and harnesses that forbid
 * hipMalloc).  Same arguments, kernels and results as loopvq_decode_attn; the split
 * partials go to a static device array of LOOPVQ_DECODE_STATIC_SCRATCH_BYTES that the
 * library holds on every GPU it runs on until the process ends (its address is looked up
 * on the first call on each device).  Nothing is allocated or freed.  A split plan that
 * needs more than the array (S * B * Hq * (d + 4) * 4 bytes with S > 1; S = 1 needs none)
 * returns LOOPVQ_ERR_WORKSPACE before any HIP call.  Every call on one GPU shares that
 * GPU's array, so calls that may overlap on one GPU (different streams, or a graph replay
 * beside another call) race; calls ordered on one stream do not.  The array needs no
 * clearing: every partial a merge reads is written by the same call. */
#define LOOPVQ_DECODE_STATIC_SCRATCH_BYTES ((size_t)16 << 20)
loopvq_status loopvq_decode_attn_noalloc(const loopvq_config* cfg, const loopvq_decode_args* args,
                                         void* stream);

/* Extend (chunked prefill): M new tokens of every sequence, whose keys and values are
 * still bf16, attend over the cached context plus the chunk itself.  The serving
 * path has a prefill backend of its own (airadar.tv summary, section
 * "Utilisation"); the pages do not describe it.  Row i of the chunk of sequence b
 * (query head hq, kv-head hq / (Hq/Hkv)) attends over every cached token exactly
 * as a decode query of the same (layer, loop step) does -- [prefix | vector-
 * quantized | recent] for N = seq_lens[b] cached tokens -- plus chunk rows 0..i
 * (causal inside the chunk), with the same softmax scale and key rotation.
 *   q            device bf16 [B][M][Hq][d]
 *   k_new, v_new device bf16 [B][Hkv][M][d]: the chunk's keys (rotated like the
 *                cache's when rot is given) and values; 16-byte aligned
 *   chunk_lens   optional device int32 [B]: rows [0, chunk_lens[b]) of sequence b
 *                are computed (others untouched); NULL = all M
 *   out          device fp32 [B][M][Hq][d]
 *   lse          optional device fp32 [B][M][Hq]: as for decode, the log-sum-exp of the row's
 *                scores, for merging this attention with other parts
 * The other fields mean what they mean for decode (windows of the same (l, t),
 * pool, rot, softmax_scale); the codebooks come in the group-major layout of
 * loopvq_codebook_prepare_groups.  No workspace is needed.  The
 * kernel dequantizes 64-token tiles into LDS.  Scores run on bf16 MFMAs (a rotated q
 * split into two bf16 parts, so fp32-level accuracy).  The value product runs on fp16
 * MFMAs with the softmax weights rounded to fp16 (relative error at most 2^-11 per
 * weight, 2^-25 absolute below 2^-14) while every value of the workgroup's tiles
 * converts to fp16 exactly (zero or magnitude in [2^-17, 2^16)); from the first tile
 * with another value on, and for the whole workgroup when the value codebook slice
 * holds one, it runs on bf16 MFMAs with the weights split into two bf16 parts
 * (2^-16 relative).  The normaliser is the sum of the weights the product used.
 * Outputs stay within the attention tolerance (rel-L2 1e-3 per row) either way. */
typedef struct loopvq_extend_args {
  int32_t layer;                /* l */
  int32_t loop;                 /* t (tau = t mod G, loop group t / G) */
  int32_t batch;                /* B */
  int32_t chunk;                /* M >= 1 */
  int32_t max_pages_per_seq;    /* as for decode */
  int32_t max_seq_len;          /* upper bound of seq_lens (cached tokens) */
  int64_t num_pages;
  const uint16_t* q;
  const uint16_t* k_new;
  const uint16_t* v_new;
  const int32_t* seq_lens;      /* device [B], each in [0, max_seq_len]; a length outside that range
                                   (which the host cannot see) is clamped to it */
  const int32_t* chunk_lens;    /* device [B] or NULL */
  const int32_t* block_table;
  const uint8_t* pool;
  const uint16_t* cb_k_grp;     /* device group-major key codebooks (loopvq_codebook_prepare_groups) */
  const uint16_t* cb_v_grp;     /* device group-major value codebooks */
  const uint16_t* k_prefix;
  const uint16_t* v_prefix;
  const uint16_t* k_recent;
  const uint16_t* v_recent;
  const float* rot;             /* [d][d] or NULL */
  float softmax_scale;          /* <= 0: 1/sqrt(d) */
  float* out;
  float* lse;                   /* device fp32 [B][M][Hq] or NULL: ln sum_n exp(scale * q'.k_n) over
                                   the keys the row sees (written for the computed rows only) */
} loopvq_extend_args;

loopvq_status loopvq_extend_attn(const loopvq_config* cfg, const loopvq_extend_args* args, void* stream);

/* Static description of a status code. */
const char* loopvq_status_string(loopvq_status s);

/* Detail of the last error on this thread ("" if none). */
const char* loopvq_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* LOOPVQ_H */
