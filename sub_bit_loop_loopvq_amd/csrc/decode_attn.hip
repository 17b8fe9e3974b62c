// LoopVQ decode attention over a packed, loop-axis vector-quantized KV cache (gfx950).
//
// What it computes (arXiv 2611.05304 abstract; airadar.tv summary, sections
// "Raisons" and "Utilisation"): one decode query of a looped transformer
// attends over [bf16 prefix rows | vector-quantized rows | bf16 recent rows].
// A vector-quantized row of loop step t stores, per channel group g, one 8-bit
// index into the (layer, kv-head, group) codebook whose codewords span the c
// channels of G consecutive loop steps; the row's channels are the
// loop-step-(t mod G) slice of that codeword.
//
// How (MI355X):
//  * one workgroup = one query x one token split.  At NG = 32 (c = 4, d = 128): 16 waves
//    and about 148 KB of LDS, one workgroup per CU; at NG = 16: 8 waves and about 72 KB,
//    two workgroups per CU.
//  * prologue: q' = scale*log2(e) * R^T q; the q.codeword lookup table
//    LUT[k][g] = q'_g . slice_tau(C_k[g]) is built in LDS (K x NG fp32).
//  * LDS layout, [0, 64K): one 256-byte row per codeword k holding LUT[k][g] at
//    byte 4*g (NG=32) or two copies at 4*g and 64 + 4*g (NG=16, so the 64 lanes
//    of a read cover all 32 banks).  [64K, 128K): the value histogram, one
//    256-byte row per codeword, H[k][g] as a 64-bit integer (slots permuted so a
//    half-wave's updates hit distinct bank pairs).  The
//    address of either entry is (region byte, index byte, group byte): one
//    v_perm_b32 merges the packed index byte with two constant bytes, so an
//    index costs one VALU op plus one LDS op.
//  * index stream: a wave reads one 1 KB block of K indices and one of V
//    indices per tile (32 tokens at NG=32, 64 at NG=16), 16 B per lane, four
//    tiles in flight.  Lane (Q, u) holds 4 tokens x 4 groups; its 16 lookups walk
//    the groups in an order rotated by Q so the lanes of one instruction hit
//    distinct banks.  Page ids of the wave's tiles are vector-loaded once and
//    read back with v_readlane.
//  * token scores: per-lane partial sums + a 2-3 step DPP reduce-scatter over
//    the lanes of a token quad, so each lane ends with one full token score.
//  * softmax: scores in log2 units; p = exp2(s - m_ref), m_ref = maximum over
//    the first tile of every wave.  A split where a later score exceeds m_ref by
//    more than 17 (log2 units) is recomputed with the exact maximum (rare).
//  * values: H[idx_V[n][g]][g] += floor(p_n * 2^30) with 64-bit LDS integer
//    atomics (exact and order independent, so the output is bitwise
//    reproducible; LDS float atomics are an order of magnitude slower on this
//    part).  Afterwards o[g*c + i] = sum_k H[k][g] * Cv_tau[k][g*c + i] and the
//    normaliser is sum_k H[k][0]: the same quantised weights.
//  * bf16 windows: a wave step reads 1 KB of K and of V rows (16 B per lane), DPP row sums
//    give the scores, and each lane accumulates p * V for its 8 channels.
//  * splits write (m, l, o) partials; a second kernel merges them with
//    log-sum-exp.  One split writes the output directly.
#include "lvq_common.h"

#include <math.h>

#include <mutex>
#include <type_traits>

// Split partials of loopvq_decode_attn_noalloc: one copy of this array lives on every GPU the
// library runs on, from module load to process end.  In host code `scratch` names a host-side
// stand-in, never the device memory: host code only uses the address hipGetSymbolAddress
// returns for the current device (lvq::decode_static_scratch).
static __device__ __align__(256) uint8_t scratch[lvq::kDecodeStaticScratchBytes];

namespace lvq {
namespace {

constexpr int kRowBytes = 256;
constexpr float kThr = 17.f;            // p <= 2^17 before a redo is forced
constexpr float kFix = 1073741824.f;    // 2^30: fixed-point scale of the histogram
constexpr float kNegInf = -INFINITY;
constexpr int kMaxTilesPerWave = 128;   // page-id vector: 2 VGPRs of 64 lanes

// Waves per workgroup.  NG=32 needs a separate 64 KB histogram region (128 KB+ of LDS, one
// workgroup per CU, 16 waves); at NG=16 the histogram fits in the unused half of the LUT
// rows (~72 KB, two workgroups per CU, 8 waves each).
template <int NG>
constexpr int waves_for() { return NG == 32 ? 16 : 8; }

template <int NG, int D, int WAVES>
struct DecodeSmem {
  uint8_t tab[kCodes * kRowBytes];              // [0, 64K): LUT rows (must stay first)
  unsigned long long hist[NG == 32 ? kCodes * 32 : 2];   // [64K, 128K) at NG=32: histogram rows
  float q[D];                                   // q' (log2 units)
  float red[2 * WAVES * 64];                    // raw q, then contraction partials
  float wo[WAVES][D];                           // window partial o per wave
  float wm[WAVES], wl[WAVES];                   // window partial max / sum per wave
  float vm0[WAVES];                             // first-tile VQ max per wave (the reference)
  float vm[WAVES];                              // VQ max per wave
  int vover[WAVES];
  float lpart[16];                              // normaliser partials of the value contraction
};

// Byte offset (from LDS address 0) of histogram entry (k, g).
template <int NG>
__device__ __forceinline__ uint32_t hist_off(uint32_t k, uint32_t g);

__device__ __forceinline__ u32x4 ntload(const u32x4* ptr) { return __builtin_nontemporal_load(ptr); }

__device__ __forceinline__ float lds_f32(const uint8_t* lds, uint32_t addr) {
  return *reinterpret_cast<const float*>(lds + addr);
}

// p in [0, 2^17] -> floor(p * 2^30) as (hi, lo) 32-bit halves, exactly
__device__ __forceinline__ void to_fixed(float p, uint32_t& hi, uint32_t& lo) {
  const float hf = floorf(p * 0.25f);                        // = floor(p * 2^30 / 2^32)
  const float lf = fmaf(hf, -4294967296.f, p * kFix);        // exact remainder in [0, 2^32)
  hi = (uint32_t)hf;
  lo = (uint32_t)lf;
}

// Slot of group g inside a 32-entry histogram row.  A 64-bit atomic touches two banks; at
// NG=32 groups g and g+16 would share a bank pair, so the slot is permuted such that the 16
// groups a half-wave of lanes updates together (4u + rr, u < 8, two consecutive rr) land on
// 16 distinct bank pairs.
template <int NG>
__device__ __forceinline__ uint32_t hist_slot(uint32_t g) {
  if constexpr (NG == 32) return 2u * (g >> 2) + (g & 1u) + 16u * ((g >> 1) & 1u);
  return g;
}

template <int NG>
__device__ __forceinline__ uint32_t hist_off(uint32_t k, uint32_t g) {
  if constexpr (NG == 32) return 65536u + k * kRowBytes + hist_slot<NG>(g) * 8u;
  return k * kRowBytes + 128u + g * 8u;
}

template <int NG, int D, int WAVES>
__device__ __forceinline__ void zero_hist(DecodeSmem<NG, D, WAVES>& sm, int tid) {
  if constexpr (NG == 32) {
    u32x4* hz = reinterpret_cast<u32x4*>(sm.hist);
    for (int e = tid; e < kCodes * 32 * 8 / 16; e += WAVES * 64) hz[e] = u32x4{0u, 0u, 0u, 0u};
  } else {
    for (int e = tid; e < kCodes * 8; e += WAVES * 64)    // 8 x 16 B per row, bytes [128, 256)
      *reinterpret_cast<u32x4*>(sm.tab + (e >> 3) * kRowBytes + 128 + (e & 7) * 16) = u32x4{0u, 0u, 0u, 0u};
  }
}

template <int NG, int C, int WAVES>
__global__ void __launch_bounds__(WAVES * 64) decode_kernel(DecodeParams p) {
  constexpr int D = NG * C;
  constexpr int G4 = NG / 4;        // lanes that share a token quad
  constexpr int TW = 256 / G4;      // tokens per wave tile (1 KB of 8-bit indices)
  constexpr int NT = WAVES * 64;
  constexpr int LPT = kCodes * NG / NT;   // LUT entries built per thread
  constexpr int NPG = kMaxTilesPerWave / 64;
  static_assert(NG == 16 || NG == 32, "NG");
  static_assert(D == 64 || D == 128, "D");
  static_assert(LPT >= 1 && NT % NG == 0, "LUT build mapping");
  using SliceT = typename std::conditional<C == 4, uint2, uint4>::type;

  __shared__ DecodeSmem<NG, D, WAVES> sm;
  uint8_t* const lds = sm.tab;      // LDS address 0

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int Q_total = p.B * p.Hq;
  const int qi = blockIdx.x / p.S;
  const int s = blockIdx.x - qi * p.S;
  const int b = qi / p.Hq;
  const int hq = qi - b * p.Hq;
  const int h = hq / (p.Hq / p.Hkv);

  // With one split, a wave's tiles are wave, wave + WAVES, ... whatever the sequence length is,
  // so their page ids are requested together with the length instead of after it (entries are
  // clamped to the block-table row; lanes past the sequence's tiles are cleared below).
  const int32_t* bt = p.block_table + (int64_t)b * p.max_pages;
  const bool pg_early = p.S == 1 && p.max_pages > 0;
  int pg_raw[NPG];
  if (pg_early) {
#pragma unroll
    for (int c = 0; c < NPG; ++c) {
      const int e = ((wave + (64 * c + lane) * WAVES) * TW) >> p.pt_shift;
      pg_raw[c] = bt[e < p.max_pages ? e : p.max_pages - 1];
    }
  }

  // N = 0 is an empty context (output 0, lse = -inf).  A length outside [0, max_seq_len] is a
  // caller error the host cannot see: the query does no work and its output row and lse are
  // written as NaN, so that it cannot pass for a result.
  int N = p.seq_lens[b];
  const bool bad_len = N < 0 || N > p.max_seq_len;
  N = bad_len ? 0 : N;
  const int n_prefix = N < p.P ? N : p.P;
  int n_vq = N - p.P - p.R;
  n_vq = n_vq < 0 ? 0 : n_vq;
  const int n_recent = N - n_prefix - n_vq;
  {
    const int cap = p.max_pages << p.pt_shift;
    if (n_vq > cap) n_vq = cap;
  }
  const int n_win = n_prefix + n_recent;
  const int w0 = (int)(((int64_t)n_win * s) / p.S);
  const int w1 = (int)(((int64_t)n_win * (s + 1)) / p.S);
  const int n_tiles = (n_vq + TW - 1) / TW;

  // bf16 window rows of this split, in wave steps of RPI rows: lane (wr, wc) holds channels
  // [8 wc, 8 wc + 8) of row wr of a step.  The wave's first step is requested here, ahead of
  // the page-id chain and the prologue, which its latency then overlaps.
  constexpr int LPR = D / 8;      // lanes per window row
  constexpr int RPI = 64 / LPR;   // rows per wave step
  const int wr = lane / LPR, wc = lane % LPR;
  const int64_t pre_row0 = ((int64_t)b * p.Hkv + h) * p.P;
  const int64_t rec_row0 = ((int64_t)b * p.Hkv + h) * p.R;
  const int wstride = WAVES * RPI;
  const int wfirst = w0 + wave * RPI;
  const int n_ws = wfirst < w1 ? (w1 - wfirst + wstride - 1) / wstride : 0;
  // (the window bases as values: a per-lane choice between two argument fields would otherwise
  // be made by loading the chosen field from the argument block, one dependent load per call)
  const uint16_t* const kpre = p.k_prefix;
  const uint16_t* const vpre = p.v_prefix;
  const uint16_t* const krec = p.k_recent;
  const uint16_t* const vrec = p.v_recent;
  auto wload = [&](int i, u32x4& kk, u32x4& vv) {   // rows past the split end re-read its last row
    int w = wfirst + i * wstride + wr;
    w = w < w1 ? w : w1 - 1;
    const bool pre = w < n_prefix;
    const int64_t off = (pre ? pre_row0 + w : rec_row0 + (w - n_prefix)) * D + 8 * wc;
    kk = ntload(reinterpret_cast<const u32x4*>((pre ? kpre : krec) + off));
    vv = ntload(reinterpret_cast<const u32x4*>((pre ? vpre : vrec) + off));
  };
  u32x4 wk0, wv0;
  if (n_ws > 0) wload(0, wk0, wv0);
  const int t0 = (int)(((int64_t)n_tiles * s) / p.S);
  const int t1 = (int)(((int64_t)n_tiles * (s + 1)) / p.S);
  const bool has_vq = t1 > t0;

  // ---- 0. issue the first global loads: page ids, the first index tiles, the key
  //         codebook slice and q, so their latency overlaps the prologue -------------
  const int Qd = lane / G4, u = lane % G4;
  // index tiles come through buffer loads over the kv-head's page region (below 2 GiB, checked
  // by the host): the tile offset is uniform (a scalar register) and each lane adds 16 B
  const uint8_t* pool_h = has_vq ? p.pool_lj + (int64_t)h * p.head_stride : p.pool_lj;
  const __amdgpu_buffer_rsrc_t pool_rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)pool_h, (short)0, 0x7fffffff, kRawBufferWord3);
  const int lane16 = lane * 16;
  const int pt_mask = (1 << p.pt_shift) - 1;
  const int my_first = t0 + wave;
  const int n_my = (has_vq && my_first < t1) ? (t1 - my_first + WAVES - 1) / WAVES : 0;

  // page ids of this wave's tiles: lane l of pg[c] holds the page of tile 64*c + l
  // (two separate paths, so that the early ids are waited for without the loads issued after
  // them)
  int pg[NPG];
  if (pg_early) {
#pragma unroll
    for (int c = 0; c < NPG; ++c) {
      const int v = pg_raw[c];
      pg[c] = (64 * c + lane < n_my && v >= 0 && v < p.num_pages) ? v : 0;
    }
  } else {
#pragma unroll
    for (int c = 0; c < NPG; ++c) {
      const int i = 64 * c + lane;
      int v = 0;
      if (i < n_my) {
        v = bt[((my_first + i * WAVES) * TW) >> p.pt_shift];
        v = (v < 0 || v >= p.num_pages) ? 0 : v;
      }
      pg[c] = v;
    }
  }
  auto tile_off = [&](int i) -> int {   // i: wave-uniform tile ordinal; byte offset in the region
    const int c = i >> 6, l = i & 63;
    int page = __builtin_amdgcn_readlane(pg[0], l);
#pragma unroll
    for (int cc = 1; cc < NPG; ++cc) {
      const int pc = __builtin_amdgcn_readlane(pg[cc], l);
      page = c == cc ? pc : page;
    }
    const int u0 = (my_first + i * WAVES) * TW;
    return page * (int)p.page_bytes + (u0 & pt_mask) * NG;
  };
  constexpr int kPF = 4;
  u32x4 bk[kPF], bv[kPF];
  auto load_first = [&]() {
#pragma unroll
    for (int j = 0; j < kPF; ++j) {
      const int to = tile_off(j < n_my ? j : n_my - 1);
      bk[j] = __builtin_amdgcn_raw_buffer_load_b128(pool_rs, lane16, to, kBufNontemporal);
      bv[j] = __builtin_amdgcn_raw_buffer_load_b128(pool_rs, lane16, to + (int)p.kind_bytes, kBufNontemporal);
    }
  };
  if (n_my > 0) load_first();

  const int g_lut = tid % NG;   // fixed per thread
  SliceT ks[LPT];
  if (has_vq) {
    const uint16_t* sk = p.cbk + ((int64_t)h * p.G + p.tau) * kCodes * D + g_lut * C;
#pragma unroll
    for (int m = 0; m < LPT; ++m) ks[m] = *reinterpret_cast<const SliceT*>(sk + ((tid + m * NT) / NG) * D);
  }
  const float qraw = tid < D ? bf16_at(p.q + (int64_t)qi * D + tid) : 0.f;

  // ---- 1. q' = scale*log2(e) * R^T q -------------------------------------------------
  if (tid < D) sm.red[tid] = qraw;
  __syncthreads();
  if (p.rot) {
    constexpr int RP = NT / D;            // partial sums per output channel
    const int j = tid % D, part = tid / D;
    float v = 0.f;
#pragma unroll 8
    for (int i = part * (D / RP); i < (part + 1) * (D / RP); ++i) v = fmaf(p.rot[i * D + j], sm.red[i], v);
    float* parts = &sm.wo[0][0];          // NT floats of scratch (window partials come later)
    parts[part * D + j] = v;
    __syncthreads();
    if (tid < D) {
      float t = 0.f;
#pragma unroll
      for (int pp = 0; pp < RP; ++pp) t += parts[pp * D + tid];
      sm.q[tid] = t * p.scale_log2;
    }
  } else if (tid < D) {
    sm.q[tid] = qraw * p.scale_log2;
  }
  __syncthreads();

  // ---- 2. lookup table and zeroed histogram ---------------------------------------------
  if (has_vq) {
    float qg[C];
#pragma unroll
    for (int i = 0; i < C; ++i) qg[i] = sm.q[g_lut * C + i];
#pragma unroll
    for (int m = 0; m < LPT; ++m) {
      const int k = (tid + m * NT) / NG;
      float acc = 0.f;
      if constexpr (C == 4) {
        const uint2 w = ks[m];
        acc = fmaf(qg[0], bf16_lo(w.x), acc);
        acc = fmaf(qg[1], bf16_hi(w.x), acc);
        acc = fmaf(qg[2], bf16_lo(w.y), acc);
        acc = fmaf(qg[3], bf16_hi(w.y), acc);
      } else {
        const uint4 w = ks[m];
        acc = fmaf(qg[0], bf16_lo(w.x), acc);
        acc = fmaf(qg[1], bf16_hi(w.x), acc);
        acc = fmaf(qg[2], bf16_lo(w.y), acc);
        acc = fmaf(qg[3], bf16_hi(w.y), acc);
        acc = fmaf(qg[4], bf16_lo(w.z), acc);
        acc = fmaf(qg[5], bf16_hi(w.z), acc);
        acc = fmaf(qg[6], bf16_lo(w.w), acc);
        acc = fmaf(qg[7], bf16_hi(w.w), acc);
      }
      float* row = reinterpret_cast<float*>(lds + k * kRowBytes);
      row[g_lut] = acc;
      if constexpr (NG == 16) row[16 + g_lut] = acc;
    }
    zero_hist(sm, tid);
  }

  // ---- 3. bf16 window rows (prefix + recent) of this split --------------------------------
  //  A wave step covers RPI rows: lane (wr, wc) loads channels [8 wc, 8 wc + 8) of row wr of
  //  the step (16 B of K and 16 B of V, so one step reads 1 KB of each), forms the partial
  //  dot product, and a DPP sum over the row's LPR lanes gives every lane its row's score.
  //  Steps are dealt to the waves round robin with four in flight per wave.  The softmax
  //  reference m_w only moves up when a score passes it by more than 8 (log2 units), so
  //  p <= 2^8 and rescaling is rare after the first step.
  float m_w = kNegInf, l_w = 0.f, o8[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) o8[c] = 0.f;
  {
    float qv[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) qv[c] = sm.q[8 * wc + c];
    auto wstep = [&](const u32x4 kk, const u32x4 vv, int i) {
      const bool live = wfirst + i * wstride + wr < w1;
      const uint32_t kw[4] = {kk.x, kk.y, kk.z, kk.w};
      float d = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        d = fmaf(qv[2 * j], bf16_lo(kw[j]), d);
        d = fmaf(qv[2 * j + 1], bf16_hi(kw[j]), d);
      }
      d += dpp<dpp_quad(1, 0, 3, 2)>(d);
      d += dpp<dpp_quad(2, 3, 0, 1)>(d);
      d += dpp<kDppRowHalfMirror>(d);
      if constexpr (LPR == 16) d += dpp<kDppRowMirror>(d);
      const float sc = live ? d : kNegInf;
      if (__builtin_amdgcn_ballot_w64(sc > m_w + 8.f) != 0) {   // first step, or a new maximum
        const float mn = fmaxf(m_w, wave_max_nolds(sc));
        const float a = __builtin_amdgcn_exp2f(m_w - mn);          // 0 on the first step
        l_w *= a;
#pragma unroll
        for (int c = 0; c < 8; ++c) o8[c] *= a;
        m_w = mn;
      }
      const float pw = live ? __builtin_amdgcn_exp2f(sc - m_w) : 0.f;
      l_w += pw;
      const uint32_t vw[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        o8[2 * j] = fmaf(pw, bf16_lo(vw[j]), o8[2 * j]);
        o8[2 * j + 1] = fmaf(pw, bf16_hi(vw[j]), o8[2 * j + 1]);
      }
    };
    if (n_ws > 0) {
      // only steps that exist are loaded (the streaming loads bypass the caches, so a
      // repeated row would be read from HBM again)
      u32x4 kb[kPF], vb[kPF];
      kb[0] = wk0;
      vb[0] = wv0;
#pragma unroll
      for (int j = 1; j < kPF; ++j)
        if (j < n_ws) wload(j, kb[j], vb[j]);
      const int n_full = n_ws - n_ws % kPF;
      for (int i0 = 0; i0 < n_full; i0 += kPF) {
#pragma unroll
        for (int j = 0; j < kPF; ++j) {
          __builtin_amdgcn_sched_barrier(0);
          wstep(kb[j], vb[j], i0 + j);
          if (i0 + j + kPF < n_ws) wload(i0 + j + kPF, kb[j], vb[j]);
        }
      }
#pragma unroll
      for (int j = 0; j < kPF - 1; ++j)
        if (n_full + j < n_ws) wstep(kb[j], vb[j], n_full + j);
    }
    // sum l and o over the wave's row groups (lanes with the same chunk wc)
    auto row_sum = [&](float v) -> float {
      if constexpr (LPR == 8) v += dpp<kDppRowRor8>(v);
      const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
      v = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
      uint32_t h0, h1;
      halves(__float_as_uint(v), h0, h1);
      return __uint_as_float(h0) + __uint_as_float(h1);
    };
    l_w = row_sum(l_w);
#pragma unroll
    for (int c = 0; c < 8; ++c) o8[c] = row_sum(o8[c]);
    // all threads finished the rotation scratch reads (barrier after q') before these writes
    if (lane == 0) {
      sm.wm[wave] = m_w;
      sm.wl[wave] = l_w;
    }
    if (lane < LPR) {
#pragma unroll
      for (int c = 0; c < 8; ++c) sm.wo[wave][8 * lane + c] = o8[c];
    }
  }

  __syncthreads();   // LUT, histogram zeroing and window partials complete

  // ---- 4. vector-quantized rows ---------------------------------------------------------
  float m_ref = kNegInf;
  if (has_vq) {
    uint32_t base_l[4], sel_l[4], base_h[4], sel_h[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t rr = (r + Qd) & 3;
      const uint32_t gg = 4u * u + rr;
      // NG=16: lanes Q and Q+4 share a group, so they read different LUT copies
      base_l[r] = gg * 4u + ((NG == 16) ? (uint32_t)((Qd >> 2) & 1) * 64u : 0u);
      sel_l[r] = 0x0c0c0000u | ((4u + rr) << 8);             // [0, 0, idx, base.b0]
      const uint32_t ho = hist_off<NG>(0, gg);                  // region and slot bytes
      base_h[r] = ho;
      sel_h[r] = (NG == 32) ? (0x0c020000u | ((4u + rr) << 8)) // [0, base.b2 = 1, idx, base.b0]
                            : (0x0c0c0000u | ((4u + rr) << 8));
    }
    const int tok = (NG == 16) ? u : (((u >= 4) ? 2 : 0) + ((u & 2) ? 1 : 0));
    const bool hi_half = (u >= 4);
    auto score = [&](const u32x4 xk, bool masked, int i) -> float {
      const uint32_t xs[4] = {xk.x, xk.y, xk.z, xk.w};
      float acc[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float a = lds_f32(lds, __builtin_amdgcn_perm(xs[j], base_l[0], sel_l[0]));
#pragma unroll
        for (int r = 1; r < 4; ++r) a += lds_f32(lds, __builtin_amdgcn_perm(xs[j], base_l[r], sel_l[r]));
        acc[j] = a;
      }
      float sc;
      if constexpr (NG == 16) {
        const bool b2 = (u & 2) != 0, b1 = (u & 1) != 0;
        const float k0 = b2 ? acc[2] : acc[0], s0 = b2 ? acc[0] : acc[2];
        const float k1 = b2 ? acc[3] : acc[1], s1 = b2 ? acc[1] : acc[3];
        const float c0 = k0 + dpp<dpp_quad(2, 3, 0, 1)>(s0);
        const float c1 = k1 + dpp<dpp_quad(2, 3, 0, 1)>(s1);
        const float kk = b1 ? c1 : c0, ss = b1 ? c0 : c1;
        sc = kk + dpp<dpp_quad(1, 0, 3, 2)>(ss);
      } else {
        const float k0 = hi_half ? acc[2] : acc[0], s0 = hi_half ? acc[0] : acc[2];
        const float k1 = hi_half ? acc[3] : acc[1], s1 = hi_half ? acc[1] : acc[3];
        const float c0 = k0 + dpp<kDppRowHalfMirror>(s0);
        const float c1 = k1 + dpp<kDppRowHalfMirror>(s1);
        const bool b2 = (u & 2) != 0;
        const float kk = b2 ? c1 : c0, ss = b2 ? c0 : c1;
        const float d0 = kk + dpp<dpp_quad(2, 3, 0, 1)>(ss);
        sc = d0 + dpp<dpp_quad(1, 0, 3, 2)>(d0);
      }
      if (masked) {
        const int pos = (my_first + i * WAVES) * TW + 4 * Qd + tok;
        sc = pos < n_vq ? sc : kNegInf;
      }
      return sc;
    };

    auto accum_v = [&](const u32x4 xv, float pp) {
      uint32_t fh, fl;
      to_fixed(pp, fh, fl);
      uint32_t ph[4], pl[4];
      if constexpr (NG == 16) {
        ph[0] = __builtin_amdgcn_mov_dpp(fh, dpp_quad(0, 0, 0, 0), 0xf, 0xf, false);
        ph[1] = __builtin_amdgcn_mov_dpp(fh, dpp_quad(1, 1, 1, 1), 0xf, 0xf, false);
        ph[2] = __builtin_amdgcn_mov_dpp(fh, dpp_quad(2, 2, 2, 2), 0xf, 0xf, false);
        ph[3] = __builtin_amdgcn_mov_dpp(fh, dpp_quad(3, 3, 3, 3), 0xf, 0xf, false);
        pl[0] = __builtin_amdgcn_mov_dpp(fl, dpp_quad(0, 0, 0, 0), 0xf, 0xf, false);
        pl[1] = __builtin_amdgcn_mov_dpp(fl, dpp_quad(1, 1, 1, 1), 0xf, 0xf, false);
        pl[2] = __builtin_amdgcn_mov_dpp(fl, dpp_quad(2, 2, 2, 2), 0xf, 0xf, false);
        pl[3] = __builtin_amdgcn_mov_dpp(fl, dpp_quad(3, 3, 3, 3), 0xf, 0xf, false);
      } else {
        // token i of the quad lives in lanes 2i, 2i+1 of the 8-lane group
        const uint32_t ah = __builtin_amdgcn_mov_dpp(fh, dpp_quad(0, 0, 0, 0), 0xf, 0xf, false);
        const uint32_t bh = __builtin_amdgcn_mov_dpp(fh, dpp_quad(2, 2, 2, 2), 0xf, 0xf, false);
        const uint32_t al = __builtin_amdgcn_mov_dpp(fl, dpp_quad(0, 0, 0, 0), 0xf, 0xf, false);
        const uint32_t bl = __builtin_amdgcn_mov_dpp(fl, dpp_quad(2, 2, 2, 2), 0xf, 0xf, false);
        const uint32_t amh = __builtin_amdgcn_mov_dpp(ah, kDppRowHalfMirror, 0xf, 0xf, false);
        const uint32_t bmh = __builtin_amdgcn_mov_dpp(bh, kDppRowHalfMirror, 0xf, 0xf, false);
        const uint32_t aml = __builtin_amdgcn_mov_dpp(al, kDppRowHalfMirror, 0xf, 0xf, false);
        const uint32_t bml = __builtin_amdgcn_mov_dpp(bl, kDppRowHalfMirror, 0xf, 0xf, false);
        ph[0] = hi_half ? amh : ah;
        ph[1] = hi_half ? bmh : bh;
        ph[2] = hi_half ? ah : amh;
        ph[3] = hi_half ? bh : bmh;
        pl[0] = hi_half ? aml : al;
        pl[1] = hi_half ? bml : bl;
        pl[2] = hi_half ? al : aml;
        pl[3] = hi_half ? bl : bml;
      }
      const uint32_t xs[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const unsigned long long v = ((unsigned long long)ph[j] << 32) | pl[j];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const uint32_t addr = __builtin_amdgcn_perm(xs[j], base_h[r], sel_h[r]);
          atomicAdd(reinterpret_cast<unsigned long long*>(lds + addr), v);
        }
      }
    };

    // reference maximum: the first tile of every wave (already in flight)
    float m_loc = kNegInf, sc_first = kNegInf;   // the first tile's scores also start pass 0
    if (n_my > 0) {
      sc_first = score(bk[0], my_first == n_tiles - 1, 0);
      m_loc = wave_max_nolds(sc_first);
    }
    if (lane == 0) sm.vm0[wave] = m_loc;   // slots of their own: no barrier before the pass reuses vm
    __syncthreads();
    m_ref = sm.vm0[0];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) m_ref = fmaxf(m_ref, sm.vm0[w]);

    for (int pass = 0; pass < 2; ++pass) {
      float smax = kNegInf;
      bool over = false;
      // Software pipeline over the wave's tiles: the key lookups of tile i are issued in the
      // same region as the value atomics of tile i-1, so each wave keeps LDS reads in flight
      // while its atomics issue; a slot is refilled once its value indices are consumed.
      auto score_of = [&](const u32x4 xk, int i) -> float {
        const bool masked = (my_first + i * WAVES) == n_tiles - 1;   // only the globally last tile is partial
        return score(xk, masked, i);
      };
      auto finish = [&](const u32x4 xv, float sc) {
        smax = fmaxf(smax, sc);
        const float e = sc - m_ref;
        over |= e > kThr;
        accum_v(xv, __builtin_amdgcn_exp2f(fminf(e, kThr)));
      };
      auto refill = [&](int slot_tile, u32x4& xk, u32x4& xv) {
        const int inext = slot_tile < n_my ? slot_tile : n_my - 1;
        const int to = tile_off(inext);
        xk = __builtin_amdgcn_raw_buffer_load_b128(pool_rs, lane16, to, kBufNontemporal);
        xv = __builtin_amdgcn_raw_buffer_load_b128(pool_rs, lane16, to + (int)p.kind_bytes, kBufNontemporal);
      };
      if (n_my > 0) {
        if (pass > 0) load_first();
        float sc_prev = pass == 0 ? sc_first : score_of(bk[0], 0);
        // steady state over tiles 1 .. n_my-1 in groups of kPF: tile i = i0 + j + 1 sits in slot
        // (j + 1) % kPF, its predecessor in slot j; refills past the end re-read the last tile
        // and are never consumed
        const int n_rest = n_my - 1;
        const int n_full = n_rest - n_rest % kPF;
        int i0 = 0;
        for (; i0 < n_full; i0 += kPF) {
#pragma unroll
          for (int j = 0; j < kPF; ++j) {
            __builtin_amdgcn_sched_barrier(0);
            const float sc = score_of(bk[(j + 1) % kPF], i0 + j + 1);
            finish(bv[j], sc_prev);
            refill(i0 + j + kPF, bk[j], bv[j]);
            sc_prev = sc;
          }
        }
#pragma unroll
        for (int j = 0; j < kPF; ++j) {
          const int i = i0 + j + 1;
          if (i < n_my) {
            const float sc = score_of(bk[(j + 1) % kPF], i);
            finish(bv[j], sc_prev);
            sc_prev = sc;
          } else if (i == n_my) {
            finish(bv[j], sc_prev);
          }
        }
      }
      smax = wave_max_nolds(smax);
      const bool wover = __any(over);
      if (lane == 0) {
        sm.vm[wave] = smax;
        sm.vover[wave] = wover ? 1 : 0;
      }
      __syncthreads();
      int any_over = 0;
      float all_max = kNegInf;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) {
        any_over |= sm.vover[w];
        all_max = fmaxf(all_max, sm.vm[w]);
      }
      if (!any_over || pass == 1) break;
      // rare: a score exceeded the reference by more than 17; redo with the exact maximum
      m_ref = all_max;
      __syncthreads();
      zero_hist(sm, tid);
      __syncthreads();
    }
  }

  // ---- 5. value contraction o_vq = H^T Cv_tau, merge, write -----------------------------
  // thread -> (channel pair cp, codeword part); each part sums KPT codewords
  constexpr int CP = D / 2;
  constexpr int PARTS = NT / CP;
  constexpr int KPT = kCodes / PARTS;
  static_assert(NT % CP == 0 && kCodes % PARTS == 0 && PARTS <= 16, "contraction mapping");
  float o_vq = 0.f, l_vq = 0.f;
  if (has_vq) {
    const int cp = tid % CP, part = tid / CP, g = (2 * cp) / C;
    const uint16_t* sv = p.cbv + ((int64_t)h * p.G + p.tau) * kCodes * D + 2 * cp;
    uint32_t cv[KPT];
#pragma unroll
    for (int m = 0; m < KPT; ++m) cv[m] = *reinterpret_cast<const uint32_t*>(sv + (part + m * PARTS) * D);
    float a0 = 0.f, a1 = 0.f, lsum = 0.f;
#pragma unroll
    for (int m = 0; m < KPT; ++m) {
      const unsigned long long hv = *reinterpret_cast<const unsigned long long*>(lds + hist_off<NG>(part + m * PARTS, g));
      const float hk = fmaf((float)(uint32_t)(hv >> 32), 4294967296.f, (float)(uint32_t)hv);
      a0 = fmaf(hk, bf16_lo(cv[m]), a0);
      a1 = fmaf(hk, bf16_hi(cv[m]), a1);
      lsum += hk;
    }
    sm.red[part * D + 2 * cp] = a0;
    sm.red[part * D + 2 * cp + 1] = a1;
    // normaliser: the quantised weights of group 0 (the same values the products used) sum to
    // l * 2^30; the thread of channel pair 0 of each part holds that part's share
    if (cp == 0) sm.lpart[part] = lsum;
  }
  __syncthreads();
  if (tid < D) {
    if (has_vq) {
#pragma unroll
      for (int pp = 0; pp < PARTS; ++pp) {
        o_vq += sm.red[pp * D + tid];
        l_vq += sm.lpart[pp];
      }
      o_vq *= 1.f / kFix;
      l_vq *= 1.f / kFix;
    }
    const bool vq_live = has_vq && l_vq > 0.f;
    float M = vq_live ? m_ref : kNegInf;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) M = fmaxf(M, sm.wm[w]);
    float lt = 0.f, ot = 0.f;
    if (M != kNegInf) {
      if (vq_live) {
        const float a = exp2f(m_ref - M);
        lt = l_vq * a;
        ot = o_vq * a;
      }
#pragma unroll
      for (int w = 0; w < WAVES; ++w) {
        if (sm.wm[w] != kNegInf) {
          const float a = exp2f(sm.wm[w] - M);
          lt = fmaf(sm.wl[w], a, lt);
          ot = fmaf(sm.wo[w][tid], a, ot);
        }
      }
    }
    if (p.S == 1) {
      const float o_fin = bad_len ? __builtin_nanf("") : (lt > 0.f ? ot / lt : 0.f);
      p.out[(int64_t)qi * D + tid] = o_fin;
      if (p.lse && tid == 0) p.lse[qi] = bad_len ? __builtin_nanf("") : M * 0.6931471805599453f + logf(lt);
    } else {
      float* wsp = p.ws + ((int64_t)s * Q_total + qi) * (D + 4);
      wsp[4 + tid] = ot;
      if (tid == 0) {
        wsp[0] = M;
        wsp[1] = lt;
      }
    }
  }
}

template <int D>
__global__ void __launch_bounds__(D) combine_kernel(DecodeParams p) {
  const int qi = blockIdx.x, tid = threadIdx.x;
  const int Q_total = p.B * p.Hq;
  float M = kNegInf;
  for (int s = 0; s < p.S; ++s) M = fmaxf(M, p.ws[((int64_t)s * Q_total + qi) * (D + 4)]);
  float lt = 0.f, ot = 0.f;
  for (int s = 0; s < p.S; ++s) {
    const float* wsp = p.ws + ((int64_t)s * Q_total + qi) * (D + 4);
    if (wsp[0] != kNegInf) {
      const float a = exp2f(wsp[0] - M);
      lt = fmaf(wsp[1], a, lt);
      ot = fmaf(wsp[4 + tid], a, ot);
    }
  }
  // the same contract as the single-split write: an empty context gives 0 and lse = -inf, a
  // length outside [0, max_seq_len] gives NaN
  const int n_seq = p.seq_lens[qi / p.Hq];
  const bool bad_len = n_seq < 0 || n_seq > p.max_seq_len;
  p.out[(int64_t)qi * D + tid] = bad_len ? __builtin_nanf("") : (lt > 0.f ? ot / lt : 0.f);
  if (p.lse && tid == 0) p.lse[qi] = bad_len ? __builtin_nanf("") : M * 0.6931471805599453f + logf(lt);
}

template <int NG, int C>
hipError_t launch_variant(const DecodeParams& p, hipStream_t stream) {
  const int Q = p.B * p.Hq;
  constexpr int W = waves_for<NG>();
  hipLaunchKernelGGL((decode_kernel<NG, C, W>), dim3(Q * p.S), dim3(W * 64), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.S == 1) return e;
  hipLaunchKernelGGL((combine_kernel<NG * C>), dim3(Q), dim3(NG * C), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t decode_static_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));   // with device `dev` current
    if (e != hipSuccess) return e;
    if (!a) return hipErrorInvalidSymbol;
    addr[dev] = a;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_decode(const DecodeParams& p, int ng, int c, hipStream_t stream) {
  if (ng == 32 && c == 4) return launch_variant<32, 4>(p, stream);
  if (ng == 16 && c == 4) return launch_variant<16, 4>(p, stream);
  if (ng == 16 && c == 8) return launch_variant<16, 8>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace lvq
