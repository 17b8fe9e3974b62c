// Shared definitions of the LoopVQ HIP library: launch parameter blocks and
// small device helpers (bf16 conversion, DPP lane exchanges).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lvq {

constexpr int kCodes = 256;     // K = 2^b for the built variant b = 8

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Parameter blocks (host fills, kernels read; passed by value)
// ---------------------------------------------------------------------------
struct DecodeParams {
  int B, Hq, Hkv, d, P, R, G;
  int pt_shift;              // log2(page_tokens)
  int max_pages;             // block-table row stride
  int max_seq_len;
  int S;                     // splits per query
  int tau;                   // loop step within its group (t mod G)
  int64_t num_pages, page_bytes, kind_bytes;
  float scale_log2;          // softmax scale * log2(e)
  const uint16_t* q;         // [B][Hq][d]
  const int32_t* seq_lens;   // [B]
  const int32_t* block_table;
  const uint8_t* pool_lj;    // pool + ((l*J + j)*Hkv) * head_stride
  int64_t head_stride;       // num_pages * page_bytes
  const uint16_t* cbk;       // prepared key codebooks of (l, jcb): [Hkv][G][K][d]
  const uint16_t* cbv;       // prepared value codebooks of (l, jcb)
  const uint16_t* k_prefix;  // [B][Hkv][P][d]
  const uint16_t* v_prefix;
  const uint16_t* k_recent;  // [B][Hkv][R][d]
  const uint16_t* v_recent;
  const float* rot;          // [d][d] or nullptr
  float* out;                // [B][Hq][d]
  float* lse;                // [B][Hq] or nullptr
  float* ws;                 // partials [S][B*Hq][d + 4] when S > 1
};

struct EncodeParams {
  // One launch covers n_slices (layer, loop group, kind) slices: one (p.layer, p.loop_group,
  // p.kind) for an encode, every slice (l, j, kind) = ((l*J + j)*2 + kind) for an eviction.
  int n_slices, layer, loop_group, kind;
  int L, J, Jcb, T;
  int n_tokens, Hkv, NG, G, pt_shift, max_pages, batch;
  int R;                     // ring slots per window (row_slot in [0, R)), eviction only
  int64_t num_pages, page_bytes, kind_bytes, head_stride;
  // sources: an encode's src points at loop step jG of its slice; an eviction's src / src_v
  // are the K / V window rings [L][T][B][Hkv][R][d]
  const uint16_t* src;
  const uint16_t* src_v;
  int64_t stride_loop, stride_token, stride_head, stride_slot;
  const int32_t* seq_id;     // [n_tokens], or nullptr: row r is sequence r
  const int32_t* vq_pos;     // [n_tokens]; a negative position skips the row
  const int32_t* row_slot;   // [n_tokens] ring slot of each row, or nullptr
  const int32_t* block_table;
  const uint16_t* cb;        // canonical codebooks [L][Jcb][Hkv][NG][K][E] read for kind 0
  const uint16_t* cb_v;      // read for kind 1 (an encode sets both to its one codebook)
  const float* norms;        // [L][Jcb][Hkv][NG][K], kind 0
  const float* norms_v;      // kind 1
  uint8_t* pool;             // pool base: [L][J][Hkv][num_pages][page_bytes]
  int32_t* out_idx;          // [n_slices][n_tokens][Hkv][NG] or nullptr
  unsigned long long* rerank_count;
};

struct ExtendParams {
  int B, Hq, Hkv, P, R, G;
  int M;                     // chunk rows per sequence (q, k_new, v_new, out stride)
  int row_blocks;            // workgroups per (sequence, kv-head): ceil(M * Hq/Hkv / 256)
  int pt_shift, max_pages, max_seq_len;
  int tau;                   // loop step within its group (t mod G)
  int64_t num_pages, page_bytes, kind_bytes, head_stride;
  float scale_log2;          // softmax scale * log2(e)
  const uint16_t* q;         // [B][M][Hq][d]
  const uint16_t* k_new;     // [B][Hkv][M][d]
  const uint16_t* v_new;
  const int32_t* seq_lens;   // [B] cached tokens before the chunk
  const int32_t* chunk_lens; // [B] or nullptr (all M)
  const int32_t* block_table;
  const uint8_t* pool_lj;    // pool + ((l*J + j)*Hkv) * head_stride, or nullptr (no VQ rows)
  const uint16_t* cbk;       // group-major key codebooks of (l, jcb): [Hkv][G][NG][K][c]
  const uint16_t* cbv;
  const uint16_t* k_prefix;  // [B][Hkv][P][d]
  const uint16_t* v_prefix;
  const uint16_t* k_recent;  // [B][Hkv][R][d]
  const uint16_t* v_recent;
  const float* rot;          // [d][d] or nullptr
  float* out;                // [B][M][Hq][d]
  float* lse;                // [B][M][Hq] or nullptr
};

struct PrepareParams {
  int64_t sets;              // L * Jcb * Hkv codebook sets
  int NG, K, c, G, d;
  const uint16_t* cb;
  uint16_t* prep;
  float* norms;
};

struct LloydParams {
  int n, Hkv, NG, G, d, E;   // samples, kv-heads, groups, loop steps, head_dim, c * G
  int chunks_a, rows_a;      // lloyd_sums: rows [chunk * rows_a, ...) per chunk
  const uint16_t* src;       // sample planes: plane tau of row r, kv-head h at
  int64_t stride_loop, stride_token, stride_head;   //  src + tau*stride_loop + r*stride_token + h*stride_head
  const float* weight;       // [n][Hkv][NG]
  const int32_t* assign;     // [n][Hkv][NG]
  uint16_t* cb;              // the set's canonical codebooks [Hkv][NG][K][E] (updated)
  float* norms;              // the set's squared norms [Hkv][NG][K] (recomputed)
  double* part_sums;         // [chunks_a][Hkv][G][d/64][K][64 channels]
  double* part_dist;         // [chunks_a][Hkv][G][NG]
  double* part_w;            // [chunks_a][Hkv][NG][K]
  double* cluster_weight;    // [Hkv][NG][K] or nullptr
  double* distortion;        // [Hkv][NG] or nullptr
};

// Launchers (defined next to their kernels).  Return hipSuccess or the launch error.
hipError_t launch_decode(const DecodeParams& p, int ng, int c, hipStream_t stream);
hipError_t launch_encode(const EncodeParams& p, int c, hipStream_t stream);
hipError_t launch_extend(const ExtendParams& p, int ng, int c, hipStream_t stream);
hipError_t launch_prepare(const PrepareParams& p, hipStream_t stream);
hipError_t launch_prepare_groups(const PrepareParams& p, hipStream_t stream);
hipError_t launch_lloyd(const LloydParams& p, int c, hipStream_t stream);

// The decode split workspace for callers that cannot allocate: a static device array of
// kDecodeStaticScratchBytes per GPU.  decode_static_scratch() returns its address on the
// current device (looked up once per device, then cached).
constexpr size_t kDecodeStaticScratchBytes = size_t(16) << 20;
hipError_t decode_static_scratch(void** ptr);

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_at(const uint16_t* p) { return __uint_as_float(uint32_t(*p) << 16); }

// DPP controls (GCN/CDNA encoding)
constexpr int dpp_quad(int a, int b, int c, int d) { return a | (b << 2) | (c << 4) | (d << 6); }
// last word of a raw (unstructured, byte-addressed) buffer resource on CDNA
constexpr int kRawBufferWord3 = 0x00020000;
// cache-policy operand of a buffer load: nontemporal (streamed once)
constexpr int kBufNontemporal = 2;
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;
constexpr int kDppRowRor8 = 0x128;   // lane i of a 16-lane row reads lane i ^ 8

// Workgroups are dispatched round-robin over the 8 XCDs, each with its own L2.  Block L runs
// on XCD L % 8; give XCD x the contiguous range of logical blocks that starts where the
// ranges of XCDs 0..x-1 end, so that an XCD works on few kv-heads (or rows) and its L2 holds what
// they share.  The map is a bijection of [0, n).
__device__ __forceinline__ int xcd_local_block(int L, int n) {
  const int x = L & 7, per = n >> 3, rem = n & 7;
  return x * per + (x < rem ? x : rem) + (L >> 3);
}

// Squared norm of one codeword of E bf16 elements, fp32, summed in element order with fused
// multiply-adds: the encode screen's seed.  Every writer of the norms uses this one routine.
__device__ __forceinline__ float codeword_norm(const uint16_t* row, int E) {
  float acc = 0.f;
  for (int e = 0; e < E; ++e) {
    const float v = bf16_at(row + e);
    acc = fmaf(v, v, acc);
  }
  return acc;
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}

// (value of half 0, value of half 1) of a wave register, in every lane
__device__ __forceinline__ void halves(uint32_t v, uint32_t& h0, uint32_t& h1) {
  const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  h0 = r[0];
  h1 = r[1];
}

// maximum over the wave without LDS: quad, half-row and row mirrors, then the row pairs and
// the wave halves
__device__ __forceinline__ float wave_max_nolds(float v) {
  v = fmaxf(v, dpp<dpp_quad(1, 0, 3, 2)>(v));
  v = fmaxf(v, dpp<dpp_quad(2, 3, 0, 1)>(v));
  v = fmaxf(v, dpp<kDppRowHalfMirror>(v));
  v = fmaxf(v, dpp<kDppRowMirror>(v));
  const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
  uint32_t h0, h1;
  halves(__float_as_uint(v), h0, h1);
  return fmaxf(__uint_as_float(h0), __uint_as_float(h1));
}

}  // namespace lvq
