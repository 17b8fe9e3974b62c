// LoopVQ encode: nearest codeword of every loop-axis sub-vector, packed into index pages (gfx950).
//
// What it computes (airadar.tv summary of LoopVQ, opening summary: the channels of
// several consecutive loop steps form one sub-vector sharing one codebook index;
// section "Raisons": indices are stored packed).  For row r, kv-head h, group g the
// sub-vector x has element tau*c + i = src[tau][r][h][g*c + i]; its index is the
// lowest k minimising ||x - C_k||^2 over the K = 256 codewords of (l, h, g).
//
// How (MI355X):
//  * workgroup = (group range, row block, kv-head); 4 waves; a wave takes one group of
//    the range at a time and up to 4 tiles of 32 rows.  The host picks the group range:
//    small batches (tokens leaving the recent window) spread groups over workgroups and
//    read their rows directly; bulk encodes give a workgroup all groups of 128 rows and
//    stage the rows in LDS, 64 channels at a time, with coalesced LDS-direct loads, so that
//    every cache line is read from HBM once.
//  * screen: S_k = ||C_k||^2 - 2 x.C_k = D_k - ||x||^2 (same order as D_k over k) for a
//    32-codeword x 32-row tile is one bf16 32x32x16 MFMA per 16 elements: the fp32
//    squared codeword norms enter as the accumulator input and the B operand is -2x
//    (exact in bf16).  Each lane holds 128 of its row's 256 values.
//  * epilogue: each value is packed with its index among the lane's 128 codewords in the
//    low 7 mantissa bits; the two smallest packed keys are kept with min3, med3 and min
//    over pairs of keys: 2.5 VALU ops per distance.  The two half-waves that share a row
//    are merged.
//  * exactness: the screen errs by at most delta = 2^-18 (||x||^2 + max_k ||C_k||^2) in
//    distance at 16 elements (2^-17 at 32) and the packing truncates by at most 2^-16
//    relative.  If the two smallest screened values are further apart than both bounds
//    allow, the screened winner is the exact argmin.  Otherwise (about one row in a thousand) the whole wave scores that row
//    against all 256 codewords as sequential fp64 sums of squared differences and keeps
//    the lowest exact minimiser (the brute-force definition).
//  * packing: the 8-bit index is stored as one byte of its 16-index micro-tile
//    (token quad x group quad) in the page the block table maps its position to.
#include "lvq_common.h"

namespace lvq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(1))) void global_void;
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// -2 times two packed finite bf16, exactly: doubling a 15-bit magnitude m adds one to the
// exponent field (m + 0x80) when it is nonzero and doubles m when it is zero (a subnormal or
// zero, where m < 0x80), i.e. adds min(m, 0x80); no half carries into the next for finite
// values.  The sign flips.
__device__ __forceinline__ uint32_t neg2_bf16x2(uint32_t w) {
  const u16x2 inc = __builtin_elementwise_min(__builtin_bit_cast(u16x2, w & 0x7fff7fffu), u16x2{0x80, 0x80});
  return (w ^ 0x80008000u) + __builtin_bit_cast(uint32_t, inc);
}

// value of a packed key with its 7 index bits cleared
__device__ __forceinline__ float key_value(float k) { return __uint_as_float(__float_as_uint(k) & 0xffffff80u); }


// channel groups per kv-head the kernels take (d / c <= 32)
constexpr int kMaxGroups = 32;

// Bulk stage: channels [ch0, ch0 + 64) of the block's rows for the G loop steps, as
// [loop step t][row r][64 channels] bf16 (128 B per row).  The 8-byte slot s (4 channels) of
// row r sits at slot s ^ ((r >> 1) & 15) of its row, so the 32 rows that a half-wave reads at
// one slot fall on 32 distinct 8-byte bank pairs.
constexpr int kStageCh = 64;
template <int ROWS>
__device__ __forceinline__ int stage_off(int r, int t, int s) {
  return (t * ROWS + r) * 128 + ((s ^ ((r >> 1) & 15)) << 3);
}

template <int C, int G, int TT, bool STAGE>
__global__ void __launch_bounds__(256, 2) encode_kernel(EncodeParams p, int groups_per_wg, int gx, int gy) {
  constexpr int E = G * C;        // sub-vector length (16 or 32)
  constexpr int NMF = E / 16;     // code MFMAs per distance tile
  constexpr int ROWS = 32 * TT;   // rows of the block
  constexpr float kDelta = E == 16 ? 0x1p-18f : 0x1p-17f;   // >= 3E 2^-24

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5, col = lane & 31;
  // logical block = (slice, kv-head, row block, group block), slice and kv-head outermost
  const int q = xcd_local_block(blockIdx.x, gridDim.x);
  const int g0 = (q % gx) * groups_per_wg;
  const int row0 = ((q / gx) % gy) * ROWS;
  const int h = (q / (gx * gy)) % p.Hkv;
  const int slice = q / (gx * gy * p.Hkv);
  const int NG = p.NG;
  int layer = p.layer, lg = p.loop_group, kind = p.kind;
  const uint16_t* src = p.src;
  if (p.n_slices > 1) {   // eviction: slice = (layer * J + loop group) * 2 + kind
    kind = slice & 1;
    lg = (slice >> 1) % p.J;
    layer = (slice >> 1) / p.J;
    src = (kind ? p.src_v : p.src) + (int64_t)(layer * p.T + lg * p.G) * p.stride_loop;
  }
  const int64_t set = ((int64_t)layer * p.Jcb + (p.Jcb > 1 ? lg : 0)) * p.Hkv + h;
  const uint16_t* cb_h = (kind ? p.cb_v : p.cb) + set * NG * kCodes * E;
  const float* nrm_h = (kind ? p.norms_v : p.norms) + set * NG * kCodes;
  uint8_t* pool_h = p.pool + ((int64_t)(layer * p.J + lg) * p.Hkv + h) * p.head_stride;
  int32_t* out_idx = p.out_idx ? p.out_idx + (int64_t)slice * p.n_tokens * p.Hkv * NG : nullptr;
  // element offset of row r (head h, loop step 0, channel 0) in src; a ring slot outside
  // [0, R) reads slot 0 (the row is then not stored)
  auto row_off = [&](int r) -> int64_t {
    int64_t o = (int64_t)r * p.stride_token + (int64_t)h * p.stride_head;
    if (p.row_slot) {
      const int sl = p.row_slot[r];
      o += (int64_t)((sl >= 0 && sl < p.R) ? sl : 0) * p.stride_slot;
    }
    return o;
  };
  const int pt_mask = (1 << p.pt_shift) - 1;
  __shared__ __align__(16) uint8_t stage[STAGE ? G * ROWS * 128 : 16];
  // rows whose screen is not conclusive, as (row in block) * 32 + group, re-ranked exactly
  // after the screen so that no wave holds up the others in the middle of it
  __shared__ uint16_t rr_list[ROWS * kMaxGroups];
  __shared__ int rr_n;
  if (threadIdx.x == 0) rr_n = 0;
  __syncthreads();

  // byte offset (within the kv-head's pool) of each row's micro-tile slot for group 0, or -1
  // when the row is past the end, its sequence or position is out of range or its page is
  // unmapped; group g adds (g / 4) * 16 + g % 4.  (All loads are issued unconditionally at
  // clamped addresses, then validated.)
  auto slot_ok = [&](int r) { return !p.row_slot || (p.row_slot[r] >= 0 && p.row_slot[r] < p.R); };
  auto slot_of = [&](int r) -> int64_t {   // the same for one row, with plain loads (re-rank)
    if (!p.pool) return -1;
    const int sq = p.seq_id ? p.seq_id[r] : r, u = p.vq_pos[r];
    if (!slot_ok(r) || sq < 0 || sq >= p.batch || u < 0 || (u >> p.pt_shift) >= p.max_pages) return -1;
    const int page = p.block_table[(int64_t)sq * p.max_pages + (u >> p.pt_shift)];
    if (page < 0 || page >= p.num_pages) return -1;
    const int w = u & pt_mask;
    return (int64_t)page * p.page_bytes + (int64_t)kind * p.kind_bytes + (w >> 2) * (NG >> 2) * 16 + (w & 3) * 4;
  };
  int64_t slot[TT];
  if (!p.pool) {   // assignment only (no pool, no positions): the indices go to out_idx alone
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) slot[tt] = -1;
  } else {
    int seq[TT], u[TT], page[TT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      const int r = min(row0 + tt * 32 + col, p.n_tokens - 1);
      seq[tt] = p.seq_id ? p.seq_id[r] : r;
      u[tt] = slot_ok(r) ? p.vq_pos[r] : -1;
    }
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      const int sq = min(max(seq[tt], 0), p.batch - 1);
      const int pg = min(max(u[tt] >> p.pt_shift, 0), p.max_pages - 1);
      page[tt] = p.block_table[(int64_t)sq * p.max_pages + pg];
    }
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      const bool ok = row0 + tt * 32 + col < p.n_tokens && seq[tt] >= 0 && seq[tt] < p.batch && u[tt] >= 0 &&
                      (u[tt] >> p.pt_shift) < p.max_pages && page[tt] >= 0 && page[tt] < p.num_pages;
      const int w = u[tt] & pt_mask;
      slot[tt] = ok ? (int64_t)page[tt] * p.page_bytes + (int64_t)kind * p.kind_bytes + (w >> 2) * (NG >> 2) * 16 +
                          (w & 3) * 4
                    : (int64_t)-1;
    }
  }

  // code tiles are fetched with buffer loads: a plain load before a loop and one in it would
  // be merged into a single load at the loop head, which undoes the prefetch
  auto cb_rsrc_of = [&](int gq) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)(cb_h + (int64_t)gq * kCodes * E), (short)0, kCodes * E * 2,
                                             kRawBufferWord3);
  };
  auto nrm_rsrc_of = [&](int gq) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)(nrm_h + gq * kCodes), (short)0, kCodes * 4, kRawBufferWord3);
  };
  // A operand rows ct*32 + col of a code tile (elements [16m + 8*half, +8)) and the tile's
  // accumulator input: register r of lane (col, half) holds the squared norm of codeword
  // ct*32 + 8*(r/4) + 4*half + r%4, the output row the 32x32 MFMA gives it
  auto fetch_code = [&](__amdgpu_buffer_rsrc_t cr, __amdgpu_buffer_rsrc_t nr, int ct, u32x4* a, f32x16& cn16) {
#pragma unroll
    for (int m = 0; m < NMF; ++m)
      a[m] = __builtin_amdgcn_raw_buffer_load_b128(cr, ((ct * 32 + col) * E + 16 * m + 8 * half) * 2, 0, 0);
    u32x4 q[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) q[i] = __builtin_amdgcn_raw_buffer_load_b128(nr, (ct * 32 + 8 * i + 4 * half) * 4, 0, 0);
    cn16 = __builtin_bit_cast(f32x16, __builtin_shufflevector(__builtin_shufflevector(q[0], q[1], 0, 1, 2, 3, 4, 5, 6, 7),
                                                              __builtin_shufflevector(q[2], q[3], 0, 1, 2, 3, 4, 5, 6, 7),
                                                              0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15));
  };
  // raw sub-vector elements [16m + 8*half, +8) of each tile's row col for group gq (direct
  // loads read the last row for rows past the end; such rows are zeroed where used)
  auto fetch_rows = [&](int gq, u32x4 (&xr)[TT][NMF]) {
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      if constexpr (STAGE) {
        const int r = tt * 32 + col;
        const int gl = gq % (kStageCh / C);   // group within the staged channels
#pragma unroll
        for (int m = 0; m < NMF; ++m) {
          uint2 lo, hi;
          if constexpr (C == 4) {             // loop steps 4m + 2*half, +1; slot gl
            lo = *reinterpret_cast<const uint2*>(stage + stage_off<ROWS>(r, 4 * m + 2 * half, gl));
            hi = *reinterpret_cast<const uint2*>(stage + stage_off<ROWS>(r, 4 * m + 2 * half + 1, gl));
          } else {                            // loop step 2m + half; slots 2gl, 2gl+1
            lo = *reinterpret_cast<const uint2*>(stage + stage_off<ROWS>(r, 2 * m + half, 2 * gl));
            hi = *reinterpret_cast<const uint2*>(stage + stage_off<ROWS>(r, 2 * m + half, 2 * gl + 1));
          }
          xr[tt][m] = u32x4{lo.x, lo.y, hi.x, hi.y};
        }
      } else {
        const uint16_t* base = src + row_off(min(row0 + tt * 32 + col, p.n_tokens - 1));
#pragma unroll
        for (int m = 0; m < NMF; ++m) {
          if constexpr (C == 4) {
            const int t0 = 4 * m + 2 * half;   // elements 16m + 8*half .. +7 = loop steps t0, t0 + 1
            const uint2 lo = *reinterpret_cast<const uint2*>(base + t0 * p.stride_loop + gq * 4);
            const uint2 hi = *reinterpret_cast<const uint2*>(base + (t0 + 1) * p.stride_loop + gq * 4);
            xr[tt][m] = u32x4{lo.x, lo.y, hi.x, hi.y};
          } else {
            const int t0 = 2 * m + half;  // elements 16m + 8*half .. +7 = loop step 2m + half
            xr[tt][m] = *reinterpret_cast<const u32x4*>(base + t0 * p.stride_loop + gq * 8);
          }
        }
      }
    }
  };
  // Fill the stage with channels [ch0, ch0 + 64) with LDS-direct dword loads: wave w copies
  // loop steps w, w + 4, ...; one instruction fills 256 consecutive stage bytes (two rows, two whole
  // 128-byte source lines), each lane fetching the source dword its stage position holds.
  // Rows past the end read the last row.
  auto stage_rows = [&](int ch0) {
    const int sl = (lane >> 1) & 15;   // stage slot of this lane
#pragma unroll
    for (int t = wave; t < G; t += 4) {
      const uint16_t* plane = src + (int64_t)t * p.stride_loop + (int64_t)h * p.stride_head;
      if (row0 + ROWS <= p.n_tokens && p.stride_token < (int64_t)1 << 30) {
        // whole block: a uniform row-pair base plus a 32-bit lane offset (which includes the
        // channel range, so that it is not kept live outside this function)
        const uint32_t lane_off = (uint32_t)half * (uint32_t)p.stride_token * 2u + (lane & 1) * 4 + ch0 * 2;
#pragma unroll 16
        for (int j = 0; j < ROWS / 2; ++j) {
          const char* rows = reinterpret_cast<const char*>(plane + (int64_t)(row0 + 2 * j) * p.stride_token);
          const uint32_t off = ((uint32_t)(sl << 3) ^ (uint32_t)((j & 15) << 3)) + lane_off;
          __builtin_amdgcn_global_load_lds((global_void*)(rows + off), (lds_void*)(stage + (t * ROWS + 2 * j) * 128),
                                           4, 0, 0);
        }
      } else {
        const uint16_t* src_l = plane + ch0 + (lane & 1) * 2;
#pragma unroll 4
        for (int j = 0; j < ROWS / 2; ++j) {
          const int row = min(row0 + 2 * j + half, p.n_tokens - 1);
          const uint16_t* src = src_l + (int64_t)row * p.stride_token + ((sl ^ (j & 15)) << 2);
          __builtin_amdgcn_global_load_lds((global_void*)src, (lds_void*)(stage + (t * ROWS + 2 * j) * 128), 4, 0,
                                           0);
        }
      }
    }
  };
  // four of the group's 256 squared codeword norms per lane (their maximum bounds the screen error)
  auto fetch_cnorms = [&](int gq, float (&cn)[4]) {
    const float* nrm_g = nrm_h + gq * kCodes;
#pragma unroll
    for (int i = 0; i < 4; ++i) cn[i] = nrm_g[lane + 64 * i];
  };

  const int gend = min(g0 + groups_per_wg, NG);
  // code tiles in flight: even tiles in A, odd tiles in B (no register copies between
  // tiles); A receives the next group's first tile during the current group's last tile
  u32x4 aA[NMF], aB[NMF];
  f32x16 nA, nB;
  if (g0 + wave < gend) fetch_code(cb_rsrc_of(g0 + wave), nrm_rsrc_of(g0 + wave), 0, aA, nA);

  // (a bulk workgroup owns all groups, so every wave passes the same staging barriers)
  for (int g = g0 + wave; g < gend; g += 4) {
    const uint16_t* cb_g = cb_h + (int64_t)g * kCodes * E;
    const __amdgpu_buffer_rsrc_t cb_rsrc = cb_rsrc_of(g);
    const __amdgpu_buffer_rsrc_t nrm_rsrc = nrm_rsrc_of(g);
    if constexpr (STAGE) {
      if (g % (kStageCh / C) < 4) {   // first group of a staged channel range
        __syncthreads();              // every wave is done with the previous range
        stage_rows((g - g % (kStageCh / C)) * C);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
      }
    }

    // ---- operands of this group's rows (rows past the end hold the last row's values and
    //      are neither stored nor re-ranked) ----
    u32x4 xb[TT][NMF];             // -2x, the B operand of the code MFMAs
    float xn[TT];                  // |x|^2 (it only enters the screen's error bound)
    float cn[4];                   // used after the screen: the loads are in flight meanwhile
    fetch_rows(g, xb);
    fetch_cnorms(g, cn);
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      float nn = 0.f;
#pragma unroll
      for (int m = 0; m < NMF; ++m)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          nn = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, xb[tt][m][w]),
                                               __builtin_bit_cast(bf16x2, xb[tt][m][w]), nn, false);
          xb[tt][m][w] = neg2_bf16x2(xb[tt][m][w]);
        }
      uint32_t n0, n1;
      halves(__float_as_uint(nn), n0, n1);
      xn[tt] = __uint_as_float(n0) + __uint_as_float(n1);
    }

    auto screen = [&](const u32x4* a, const f32x16& cn16, const u32x4* xs) -> f32x16 {
      f32x16 acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[0]), as_bf16x8(xs[0]), cn16, 0, 0, 0);
#pragma unroll
      for (int m = 1; m < NMF; ++m)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[m]), as_bf16x8(xs[m]), acc, 0, 0, 0);
      return acc;
    };

    // ---- screen: 8 tiles of 32 codewords; keep the two smallest packed keys per lane ----
    // key = S bits with the low 7 mantissa bits replaced by the index j = 16 ct + r of the
    // value within the lane's 128 codewords (register r of tile ct holds codeword
    // 32 ct + 8 (r / 4) + 4 half + r % 4).  Clearing low mantissa bits moves a value towards
    // zero, which keeps the order of distinct truncated values; keys with equal truncated
    // values are never told apart without the exact re-rank.  Keys are taken two at a time:
    // the new minimum is min3(b1, k0, k1) and the new second minimum is min(b2, med3(b1, k0,
    // k1)) (if b2 stays among the two smallest, b1 is the smallest and both keys are >= b2;
    // otherwise the two smallest are among b1, k0, k1 and med3 is the larger of them).  Keys
    // are finite and never NaN, so no canonicalisation is needed.
    float b1[TT], b2[TT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      b1[tt] = INFINITY;
      b2[tt] = INFINITY;
    }
    // the key mask in a register (as a literal it would split each pack into two ops)
    uint32_t keep;
    asm("v_mov_b32 %0, %1" : "=v"(keep) : "s"(0xffffff80u));
    auto consume = [&](const f32x16 (&acc)[TT], int ct) {
      // first index of the tile, hidden from the optimiser: with known low bits it would
      // split each pack into an and plus an add
      uint32_t ctb;
      asm("s_mov_b32 %0, %1" : "=s"(ctb) : "s"(ct * 16));
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          // index of register r in this lane's codeword set
          const uint32_t kl = ctb + r;
          const float k0 = __uint_as_float((__float_as_uint(acc[tt][r]) & keep) | kl);
          const float k1 = __uint_as_float((__float_as_uint(acc[tt][r + 1]) & keep) | (kl + 1));
          // (plain VALU operands only: the MFMA results are read by the compiled pack above,
          // whose wait states the compiler inserts)
          float t;
          asm("v_med3_f32 %2, %0, %3, %4\n\t"
              "v_min3_f32 %0, %0, %3, %4\n\t"
              "v_min_f32 %1, %1, %2"
              : "+v"(b1[tt]), "+v"(b2[tt]), "=&v"(t)
              : "v"(k0), "v"(k1));
        }
      }
    };
#pragma unroll 1
    for (int ct = 0; ct < kCodes / 32; ct += 2) {
      fetch_code(cb_rsrc, nrm_rsrc, ct + 1, aB, nB);
      {
        f32x16 acc[TT];
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) acc[tt] = screen(aA, nA, xb[tt]);
        consume(acc, ct);
        // the tile after next, or the next group's first tile (this group's first after the
        // last group), arrives while tile ct + 1 is finished.  The load is unconditional, so
        // that the wait before tile ct + 1 counts only the loads of B.
        const bool more = ct + 2 < kCodes / 32;
        const bool next_g = !more && g + 4 < gend;
        fetch_code(more ? cb_rsrc : (next_g ? cb_rsrc_of(g + 4) : cb_rsrc),
                   more ? nrm_rsrc : (next_g ? nrm_rsrc_of(g + 4) : nrm_rsrc), more ? ct + 2 : 0, aA, nA);
      }
      {
        f32x16 acc[TT];
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) acc[tt] = screen(aB, nB, xb[tt]);
        consume(acc, ct + 1);
      }
    }

    // ---- merge the two half-waves and decide ----
    // largest squared codeword norm of this group (for the screen's error bound)
    const float cmax = wave_max_nolds(fmaxf(fmaxf(cn[0], cn[1]), fmaxf(cn[2], cn[3])));
    uint32_t best[TT];
    bool rerank[TT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      const bool ok = row0 + tt * 32 + col < p.n_tokens;
      // both halves' two smallest keys in every lane (codeword = local index + 4 * half);
      // where the smallest truncated values are equal, either index may be taken: the gap is
      // then zero and the row is re-ranked
      uint32_t p1, q1, p2, q2;
      halves(__float_as_uint(b1[tt]), p1, q1);
      halves(__float_as_uint(b2[tt]), p2, q2);
      const float u1 = key_value(__uint_as_float(p1)), w1 = key_value(__uint_as_float(q1));
      const float u2 = key_value(__uint_as_float(p2)), w2 = key_value(__uint_as_float(q2));
      const uint32_t j1 = w1 < u1 ? q1 & 0x7fu : p1 & 0x7fu;
      const uint32_t k1 = ((j1 & ~3u) << 1) + (j1 & 3u) + (w1 < u1 ? 4u : 0u);
      const float d1 = fminf(u1, w1);                                        // screened D - |x|^2
      const float d2 = fminf(fmaxf(u1, w1), fminf(u2, w2));                  // runner-up
      // screen error bound: with sequential fp32 sums, E roundings in the products' sum
      // (whose terms total at most |x|^2 + 2|C|^2) and E - 1 in the codeword norm, i.e. at
      // most 3E 2^-24 (|x|^2 + |C|^2); 2^-100 covers flushed subnormal products
      const float delta = kDelta * (xn[tt] + cmax) + 0x1p-100f;
      const float trunc = 0x1p-15f * fmaxf(fabsf(d1), fabsf(d2));   // two keys, 2^-16 each
      rerank[tt] = ok && !(d2 - d1 > 2.f * delta + trunc);
      best[tt] = k1;
    }

    // ---- rows whose screen is not conclusive go to the exact re-rank list ----
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      if (rerank[tt] && half == 0) {
        const int e = atomicAdd(&rr_n, 1);
        rr_list[e] = (uint16_t)(((tt * 32 + col) << 5) | g);
      }
    }

    // ---- store ----
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      const int r = row0 + tt * 32 + col;
      if (half == 0 && r < p.n_tokens && !rerank[tt]) {
        if (out_idx) out_idx[((int64_t)r * p.Hkv + h) * NG + g] = (int)best[tt];
        if (slot[tt] >= 0) pool_h[slot[tt] + (g >> 2) * 16 + (g & 3)] = (uint8_t)best[tt];
      }
    }
  }

  // ---- exact re-rank of the listed rows: for each, the whole wave scores all 256 codewords,
  //      4 per lane, as fp64 sums of squared differences taken in element order with a
  //      separate rounding of every product and sum (the brute-force definition, no fused
  //      operations), and keeps the lowest index among the minimisers ----
  __syncthreads();
  const int nrr = rr_n;
  for (int e = wave; e < nrr; e += 4) {
    const int ent = __builtin_amdgcn_readfirstlane((int)rr_list[e]);
    const int gq = ent & 31, rl = ent >> 5;
    const int r = row0 + rl;
    // the row's elements tau*c + i = src[tau][r][h][gq*c + i], two per word (uniform loads)
    uint32_t xw[E / 2];
#pragma unroll
    for (int t = 0; t < G; ++t) {
      const uint32_t* xs = reinterpret_cast<const uint32_t*>(src + row_off(r) + (int64_t)t * p.stride_loop + gq * C);
#pragma unroll
      for (int i = 0; i < C / 2; ++i) xw[t * (C / 2) + i] = xs[i];
    }
    const uint16_t* cb_q = cb_h + (int64_t)gq * kCodes * E;
    // the lane's four codewords lane + 64 i, loaded together; four independent sums
    u32x4 cv[kCodes / 64][E / 8];
#pragma unroll
    for (int i = 0; i < kCodes / 64; ++i)
#pragma unroll
      for (int e8 = 0; e8 < E / 8; ++e8) cv[i][e8] = reinterpret_cast<const u32x4*>(cb_q + (lane + 64 * i) * E)[e8];
    double bd = INFINITY;
    uint32_t bk = 0u;
#pragma unroll
    for (int i = 0; i < kCodes / 64; ++i) {
      double dd = 0.0;
      {
#pragma clang fp contract(off)
#pragma unroll
        for (int e2 = 0; e2 < E / 2; ++e2) {
          const uint32_t cw = cv[i][e2 >> 2][e2 & 3];
          const double d0 = (double)bf16_lo(xw[e2]) - (double)bf16_lo(cw);
          dd = dd + d0 * d0;
          const double d1 = (double)bf16_hi(xw[e2]) - (double)bf16_hi(cw);
          dd = dd + d1 * d1;
        }
      }
      if (dd < bd) {   // k grows with i: a strict comparison keeps the lowest index
        bd = dd;
        bk = (uint32_t)(lane + 64 * i);
      }
    }
    // wave minimum of (distance, index)
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const double od = __shfl_xor(bd, off, 64);
      const uint32_t ok2 = __shfl_xor(bk, off, 64);
      if (od < bd || (od == bd && ok2 < bk)) {
        bd = od;
        bk = ok2;
      }
    }
    if (lane == 0) {
      if (out_idx) out_idx[((int64_t)r * p.Hkv + h) * NG + gq] = (int)bk;
      const int64_t sl = slot_of(r);
      if (sl >= 0) pool_h[sl + (gq >> 2) * 16 + (gq & 3)] = (uint8_t)bk;
      if (p.rerank_count) atomicAdd(p.rerank_count, 1ull);
    }
  }
}

}  // namespace

hipError_t launch_encode(const EncodeParams& p, int c, hipStream_t stream) {
  if (p.n_tokens == 0) return hipSuccess;
  // small batches (tokens leaving the recent window): one group per wave, spread over many
  // workgroups; bulk: a workgroup owns every group of 128 rows, so each cache row is read
  // whole by one workgroup
  // (an eviction's rows sit at ring slots, not at a fixed row stride: always the direct path)
  const bool small = p.n_slices > 1 || (int64_t)p.n_tokens * p.Hkv < 16384;
  // bulk rows per workgroup: the stage holds G loop steps of 64 channels per row
  const int bulk_rows = p.G == 8 ? 64 : 128;
  const int groups_per_wg = small ? 4 : p.NG;
  const int rows_per_wg = small ? 64 : bulk_rows;
  const int gx = (p.NG + groups_per_wg - 1) / groups_per_wg;
  const int gy = (p.n_tokens + rows_per_wg - 1) / rows_per_wg;
  const int64_t blocks = (int64_t)gx * gy * p.Hkv * p.n_slices;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks);
  // the staged bulk path takes 64 channels at a time
  if (!small && (p.NG * c) % kStageCh != 0) return hipErrorInvalidValue;
  if (p.NG > kMaxGroups) return hipErrorInvalidValue;
#define LVQ_ENCODE(C_, G_, TT_, ST_) \
  hipLaunchKernelGGL((encode_kernel<C_, G_, TT_, ST_>), grid, dim3(256), 0, stream, p, groups_per_wg, gx, gy)
  if (c == 4 && p.G == 4) {
    if (small) LVQ_ENCODE(4, 4, 2, false); else LVQ_ENCODE(4, 4, 4, true);
  } else if (c == 8 && p.G == 4) {
    if (small) LVQ_ENCODE(8, 4, 2, false); else LVQ_ENCODE(8, 4, 4, true);
  } else if (c == 8 && p.G == 2) {
    if (small) LVQ_ENCODE(8, 2, 2, false); else LVQ_ENCODE(8, 2, 4, true);
  } else if (c == 4 && p.G == 8) {
    if (small) LVQ_ENCODE(4, 8, 2, false); else LVQ_ENCODE(4, 8, 2, true);
  } else {
    return hipErrorInvalidValue;
  }
#undef LVQ_ENCODE
  return hipGetLastError();
}

}  // namespace lvq
