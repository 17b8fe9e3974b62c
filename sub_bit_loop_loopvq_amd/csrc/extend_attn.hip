// LoopVQ extend (chunked prefill) attention over the packed, loop-axis vector-quantized cache (gfx950).
//
// What it computes (airadar.tv summary of LoopVQ, section "Utilisation": the serving path
// keeps P prefix and R recent tokens in bf16 and has its own prefill backend; section
// "Raisons": indices are stored packed).  For one (layer, loop step), chunk row i of
// sequence b (query head hq, kv-head h = hq / (Hq / Hkv)) attends over every cached token,
// [bf16 prefix | vector-quantized rows | bf16 recent] exactly as a decode query does, plus the
// chunk's own bf16 rows 0..i.  A vector-quantized row's channels g*c .. g*c+c-1 are the
// loop-step-tau slice of codeword idx[n][g] of (layer, kv-head, group g).
//
// How (MI355X):
//  * workgroup = 128 query rows (row = (chunk token, q-head of the kv-head)) of one
//    (sequence, kv-head); 4 waves of 32 rows.  Keys come in tiles of 64 tokens.
//  * each tile is staged in LDS by the whole workgroup: K as [token][d] bf16 rows and V
//    transposed as [d][token] bf16 (rows padded so the MFMA operand reads hit distinct banks).
//    Vector-quantized tokens are dequantized on the way: the packed index byte of (token,
//    group) selects the c channels of that group's loop-step slice, read from the group-major
//    codebook copy ([tau][g][k][i]), so a tile's gathers of one group stay within K x c
//    elements (2 KB at c=4) and share cache lines.
//  * per wave: S^T = K Q^T on bf16 32x32x16 MFMAs (a rotated q' = R^T q is split into two
//    bf16 parts, two MFMAs), online softmax in log2 units with the causal mask of the
//    chunk, then O^T += V^T P^T with P split into two bf16 parts (hi + lo, 2^-16 relative),
//    so the products keep fp32-level accuracy.  The D-layout of S^T (lane = query row,
//    registers = tokens) is directly the B operand of the second product once its 16
//    tokens are taken in the order the registers hold them; the V^T operand reads the same
//    order.
#include "lvq_common.h"

namespace lvq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kKT = 64;        // keys per tile
constexpr int kVRow = kKT + 4; // bf16 per transposed V row (8 B of padding)

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// round-to-nearest-even fp32 -> bf16 bits (finite inputs)
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}
// v -> bf16 pair (hi, lo) with hi + lo == v to 2^-16 relative
__device__ __forceinline__ void split2(float v, uint32_t& hi, uint32_t& lo) {
  hi = bf16_rne(v);
  lo = bf16_rne(v - __uint_as_float(hi << 16));
}

template <int NG, int C, bool ROT>
__global__ void __launch_bounds__(ROT ? 256 : 512, ROT ? 2 : 1) extend_kernel(ExtendParams p) {
  // Without a rotation: 8 waves (256 query rows) per workgroup, one workgroup per CU, so each
  // staged tile serves twice the rows; with one, 4 waves and two workgroups per CU.
  constexpr int NTH = ROT ? 256 : 512;
  constexpr int kRows = NTH / 2;
  constexpr int D = NG * C;
  constexpr int KROW = D + 8;         // bf16 per K row (16 B of padding)
  constexpr int KSTEPS = D / 16;      // k-steps of S^T = K Q^T
  constexpr int DB = D / 32;          // 32-channel blocks of O^T
  // Without a rotation the q operand lives in LDS (each wave reads back only its own rows), which
  // frees the registers that hold the next tile's keys and values while this one is consumed.
  constexpr bool QL = !ROT;
  constexpr int QROW = D + 8;         // bf16 per q row (16 B of padding)
  // K / V^T tiles: two buffers without a rotation (tile k + 1 is staged while tile k is consumed)
  __shared__ __align__(16) uint16_t ks2[QL ? 2 : 1][kKT * KROW];
  __shared__ __align__(16) uint16_t vt2[QL ? 2 : 1][D * kVRow];
  uint16_t* ks = ks2[0];
  uint16_t* vt = vt2[0];
  __shared__ __align__(16) uint16_t qs[QL ? kRows * QROW : 8];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, col = lane & 31;
  const int grp = p.Hq / p.Hkv;
  const int rb = blockIdx.x % p.row_blocks;
  const int bh = blockIdx.x / p.row_blocks;
  const int h = bh % p.Hkv, b = bh / p.Hkv;

  // context split of the cached tokens (as in decode) and this sequence's chunk length
  int N = p.seq_lens[b];
  N = N < 0 ? 0 : (N > p.max_seq_len ? p.max_seq_len : N);
  const int n_prefix = N < p.P ? N : p.P;
  int n_vq = N - p.P - p.R;
  n_vq = n_vq < 0 ? 0 : n_vq;
  if (n_vq > (p.max_pages << p.pt_shift)) n_vq = p.max_pages << p.pt_shift;
  const int n_recent = N - n_prefix - n_vq;
  int Mb = p.chunk_lens ? p.chunk_lens[b] : p.M;
  Mb = Mb < 0 ? 0 : (Mb > p.M ? p.M : Mb);

  const int row_ws = rb * kRows;                  // first row of the workgroup
  if (row_ws / grp >= Mb) return;                 // no active row (uniform over the workgroup)
  const int i_last = min(Mb - 1, (row_ws + kRows - 1) / grp);

  // ---- this lane's query row and its q operand (B of S^T = K Q^T) --------------------------
  const int row = row_ws + wave * 32 + col;
  const int qi = row / grp;                       // chunk token of the row
  const int hq = h * grp + row % grp;
  const bool active = qi < Mb;
  const uint16_t* qrow = p.q + (((int64_t)b * p.M + (active ? qi : 0)) * p.Hq + hq) * D;
  u32x4 bq[KSTEPS], bq_lo[KSTEPS];
  if constexpr (ROT) {
    // q' = R^T q in fp32 for the 8 channels 16kk + 8*half + j this lane supplies, split in two
#pragma unroll 1
    for (int kk = 0; kk < KSTEPS; ++kk) {
      float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      const int d0 = 16 * kk + 8 * half;
#pragma unroll 4
      for (int e = 0; e < D; ++e) {
        const float qe = bf16_at(qrow + e);
        const float* re = p.rot + (int64_t)e * D + d0;
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = fmaf(re[j], qe, acc[j]);
      }
      uint32_t hi[8], lo[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) split2(acc[j], hi[j], lo[j]);
      bq[kk] = u32x4{hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16), hi[4] | (hi[5] << 16), hi[6] | (hi[7] << 16)};
      bq_lo[kk] = u32x4{lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16), lo[4] | (lo[5] << 16), lo[6] | (lo[7] << 16)};
    }
  } else {
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(qrow + 16 * kk + 8 * half);
      if constexpr (QL) {
        *reinterpret_cast<u32x4*>(qs + (wave * 32 + col) * QROW + 16 * kk + 8 * half) = v;
      } else {
        bq[kk] = v;
        bq_lo[kk] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};
  float m_ref = -INFINITY, l_run = 0.f;

  const int64_t bhk = (int64_t)b * p.Hkv + h;
  const uint8_t* pool_h = p.pool_lj ? p.pool_lj + (int64_t)h * p.head_stride : nullptr;
  const int pt_mask = (1 << p.pt_shift) - 1;
  const uint16_t* slice_k = p.cbk ? p.cbk + ((int64_t)h * p.G + p.tau) * kCodes * D : nullptr;
  const uint16_t* slice_v = p.cbv ? p.cbv + ((int64_t)h * p.G + p.tau) * kCodes * D : nullptr;

  // ---- key tiles -----------------------------------------------------------------------------
  // Tile k of this workgroup: prefix tiles, vector-quantized tiles, recent tiles, then the
  // chunk's tiles up to the workgroup's last row.  A tile's packed indices are fetched while the
  // previous tile is consumed; its keys are then gathered, written to LDS and consumed.  (Two
  // workgroups share a CU, so one's staging overlaps the other's products.)
  const int t_pre = (n_prefix + kKT - 1) / kKT, t_vq = (n_vq + kKT - 1) / kKT, t_rec = (n_recent + kKT - 1) / kKT;
  const int t_ch = i_last / kKT + 1;
  const int n_tiles = t_pre + t_vq + t_rec + t_ch;
  struct Tile {
    int seg, start, count;    // seg 0 prefix, 1 vector-quantized, 2 recent, 3 chunk
  };
  auto tile_of = [&](int k) -> Tile {
    if (k < t_pre) return {0, k * kKT, n_prefix - k * kKT};
    k -= t_pre;
    if (k < t_vq) return {1, k * kKT, n_vq - k * kKT};
    k -= t_vq;
    if (k < t_rec) return {2, k * kKT, n_recent - k * kKT};
    k -= t_rec;
    return {3, k * kKT, i_last + 1 - k * kKT};
  };
  const uint16_t* k_seg[4] = {p.k_prefix + bhk * p.P * D, nullptr, p.k_recent + bhk * p.R * D, p.k_new + bhk * p.M * D};
  const uint16_t* v_seg[4] = {p.v_prefix + bhk * p.P * D, nullptr, p.v_recent + bhk * p.R * D, p.v_new + bhk * p.M * D};

  constexpr int PIECES = D / 8;                     // 16-byte pieces per bf16 row
  constexpr int RITEMS = kKT * PIECES / NTH;        // row pieces per thread
  constexpr int QIT = kKT * (NG / 4);               // (token, group quad) items of a tile
  constexpr int QITEMS = (QIT + NTH - 1) / NTH;     // per thread (the last may be idle)
  constexpr bool kAllLive = QIT % NTH == 0;
  static_assert(RITEMS >= 1 && RITEMS * NTH == kKT * PIECES && QITEMS >= 1, "tile mapping");
  constexpr int FB = RITEMS * 4 > QITEMS * 4 * (C / 2) ? RITEMS * 4 : QITEMS * 4 * (C / 2);   // dwords per kind
  uint32_t fk[FB], fv[FB];          // the tile's keys / values on their way to LDS
  uint32_t ik_n[QITEMS], iv_n[QITEMS];   // packed indices of the next tile
  bool ok_n[QITEMS];

  // packed indices of a vector-quantized tile (token quads x group quads of one page: the tile
  // is 64 aligned positions and a page holds a power of two >= 64, so one page per tile).  All
  // loads are unconditional at clamped addresses; ok[] marks the real entries.
  auto fetch_idx = [&](int k, uint32_t* ik, uint32_t* iv, bool* ok) {
    const Tile tl = tile_of(k);
    if (tl.seg != 1) return;
    int page = p.block_table[(int64_t)b * p.max_pages + (tl.start >> p.pt_shift)];
    const bool pok = page >= 0 && page < p.num_pages;
    page = pok ? page : 0;
#pragma unroll
    for (int m = 0; m < QITEMS; ++m) {
      const int it0 = tid + NTH * m;
      const bool live = kAllLive || it0 < QIT;
      const int it = live ? it0 : 0;
      const int t = it % kKT, gq = it / kKT;
      ok[m] = live && pok && t < tl.count;
      const int w = (tl.start + min(t, tl.count - 1)) & pt_mask;
      const uint8_t* tile = pool_h + (int64_t)page * p.page_bytes + (((w >> 2) * (NG / 4) + gq) * 16 + (w & 3) * 4);
      ik[m] = *reinterpret_cast<const uint32_t*>(tile);
      iv[m] = *reinterpret_cast<const uint32_t*>(tile + p.kind_bytes);
    }
  };
  bool ok_cur[QITEMS];   // ok flags of the tile whose keys are in fk / fv
  // keys / values of tile k into registers (vector-quantized rows from their indices); rows past
  // the tile's count read the last valid row and are zeroed by store()
  auto fetch = [&](int k, const uint32_t* ik, const uint32_t* iv, const bool* ok) {
    const Tile tl = tile_of(k);
    if (tl.seg == 1) {
#pragma unroll
      for (int m = 0; m < QITEMS; ++m) {
        ok_cur[m] = ok[m];
        const int it0 = tid + NTH * m;
        const int gq = (kAllLive || it0 < QIT ? it0 : 0) / kKT;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int g = 4 * gq + r;
          const uint32_t kx = (ik[m] >> (8 * r)) & 0xffu, vx = (iv[m] >> (8 * r)) & 0xffu;
          const uint32_t* kc = reinterpret_cast<const uint32_t*>(slice_k + (g * kCodes + kx) * C);
          const uint32_t* vc = reinterpret_cast<const uint32_t*>(slice_v + (g * kCodes + vx) * C);
#pragma unroll
          for (int e = 0; e < C / 2; ++e) {
            fk[(m * 4 + r) * (C / 2) + e] = kc[e];
            fv[(m * 4 + r) * (C / 2) + e] = vc[e];
          }
        }
      }
    } else {
      const uint16_t* kw = (tl.seg == 0 ? k_seg[0] : tl.seg == 2 ? k_seg[2] : k_seg[3]) + (int64_t)tl.start * D;
      const uint16_t* vw = (tl.seg == 0 ? v_seg[0] : tl.seg == 2 ? v_seg[2] : v_seg[3]) + (int64_t)tl.start * D;
#pragma unroll
      for (int m = 0; m < RITEMS; ++m) {
        const int it = tid + NTH * m;
        const int t = min(it / PIECES, tl.count - 1), pc = it % PIECES;
        const u32x4 kv = *reinterpret_cast<const u32x4*>(kw + (int64_t)t * D + 8 * pc);
        const u32x4 vv = *reinterpret_cast<const u32x4*>(vw + (int64_t)t * D + 8 * pc);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          fk[4 * m + w] = kv[w];
          fv[4 * m + w] = vv[w];
        }
      }
    }
  };
  // the registers of tile k into LDS: K as [token][d], V transposed [d][token]; entries past the
  // tile's keys are written as zeros
  auto store = [&](int k) {
    const Tile tl = tile_of(k);
    if (tl.seg == 1) {
#pragma unroll
      for (int m = 0; m < QITEMS; ++m) {
        const int it = tid + NTH * m;
        if (!kAllLive && it >= QIT) continue;
        const int t = it % kKT, gq = it / kKT;
        const uint32_t keep = ok_cur[m] ? 0xffffffffu : 0u;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int g = 4 * gq + r;
          uint32_t* kd = reinterpret_cast<uint32_t*>(ks + t * KROW + g * C);
#pragma unroll
          for (int e = 0; e < C / 2; ++e) {
            const uint32_t vw = fv[(m * 4 + r) * (C / 2) + e] & keep;
            kd[e] = fk[(m * 4 + r) * (C / 2) + e] & keep;
            vt[(g * C + 2 * e) * kVRow + t] = (uint16_t)(vw & 0xffffu);
            vt[(g * C + 2 * e + 1) * kVRow + t] = (uint16_t)(vw >> 16);
          }
        }
      }
    } else {
#pragma unroll
      for (int m = 0; m < RITEMS; ++m) {
        const int it = tid + NTH * m;
        const int t = it / PIECES, pc = it % PIECES;
        const uint32_t keep = t < tl.count ? 0xffffffffu : 0u;
        *reinterpret_cast<u32x4*>(ks + t * KROW + 8 * pc) =
            u32x4{fk[4 * m] & keep, fk[4 * m + 1] & keep, fk[4 * m + 2] & keep, fk[4 * m + 3] & keep};
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t vw = fv[4 * m + w] & keep;
          vt[(8 * pc + 2 * w) * kVRow + t] = (uint16_t)(vw & 0xffffu);
          vt[(8 * pc + 2 * w + 1) * kVRow + t] = (uint16_t)(vw >> 16);
        }
      }
    }
  };

  // ---- one staged tile: scores, online softmax, value products --------------------------------
  // chunk_j0 >= 0 marks chunk keys: key t is chunk token chunk_j0 + t (causal); count = valid keys.
  // Rows past the chunk length compute on row 0's q and are never written, so they need no mask.
  // The softmax reference m_ref (log2 units) moves only when a score exceeds it by more than
  // 8: exponentials stay <= 2^8 and o, l are rescaled rarely.
  const float cl2 = p.scale_log2;
  auto consume = [&](int count, int chunk_j0) {
    f32x16 s[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      // all of the block's K operands first, so the LDS reads overlap instead of each MFMA
      // waiting for its own
      u32x4 a[KSTEPS];
      const uint16_t* krow = ks + (32 * mb + col) * KROW + 8 * half;
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) a[kk] = *reinterpret_cast<const u32x4*>(krow + 16 * kk);
      f32x16 acc = {};
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) {
        const u32x4 qb = QL ? *reinterpret_cast<const u32x4*>(qs + (wave * 32 + col) * QROW + 16 * kk + 8 * half)
                            : bq[kk];
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[kk]), as_bf16x8(qb), acc, 0, 0, 0);
        if constexpr (ROT)
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[kk]), as_bf16x8(bq_lo[kk]), acc, 0, 0, 0);
      }
      s[mb] = acc;
    }
    // raw scores; token of register r of block mb: 32mb + 8(r/4) + 4half + r%4
    if (count < kKT || chunk_j0 >= 0) {   // (uniform) a tile with keys to hide
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int t = 32 * mb + 8 * (r >> 2) + 4 * half + (r & 3);
          const bool vis = t < count && (chunk_j0 < 0 || chunk_j0 + t <= qi);
          s[mb][r] = vis ? s[mb][r] : -INFINITY;
        }
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, s[mb][r]);
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64)) * cl2;
    const bool move = tmax > m_ref + 8.f;       // m_ref = -inf: any visible key moves it
    if (__builtin_amdgcn_ballot_w64(move)) {
      const float alpha = move ? __builtin_amdgcn_exp2f(m_ref - tmax) : 1.f;   // m_ref = -inf -> 0
      m_ref = move ? tmax : m_ref;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
    }
    // (a row with nothing visible yet keeps m_ref = -inf and uses 0, so exp2(-inf) = 0)
    const float nm = m_ref == -INFINITY ? 0.f : -m_ref;
    float psum = 0.f;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = __builtin_amdgcn_exp2f(fmaf(s[mb][r], cl2, nm));
        s[mb][r] = e;
        psum += e;
      }
    l_run += psum;
    // O^T += V^T P^T over 4 k-steps of 16 keys; P = hi + lo with hi the truncated upper half and
    // lo = P - hi (exact) rounded to bf16 by the hardware conversion: 2^-16 relative
#pragma unroll
    for (int kst = 0; kst < kKT / 16; ++kst) {
      const int mb = kst >> 1, r0 = 8 * (kst & 1);
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t ua = __float_as_uint(s[mb][r0 + 2 * j]), ub = __float_as_uint(s[mb][r0 + 2 * j + 1]);
        hw[j] = __builtin_amdgcn_perm(ub, ua, 0x07060302u);
        const f32x2 lo = {__uint_as_float(ua) - __uint_as_float(ua & 0xffff0000u),
                          __uint_as_float(ub) - __uint_as_float(ub & 0xffff0000u)};
        lw[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf16x2));
      }
      const u32x4 bh = {hw[0], hw[1], hw[2], hw[3]};
      const u32x4 bl = {lw[0], lw[1], lw[2], lw[3]};
      u32x4 a[DB];
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const uint16_t* vrow = vt + (32 * db + col) * kVRow + 16 * kst + 4 * half;
        const uint2 v0 = *reinterpret_cast<const uint2*>(vrow);
        const uint2 v1 = *reinterpret_cast<const uint2*>(vrow + 8);
        a[db] = u32x4{v0.x, v0.y, v1.x, v1.y};
      }
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[db]), as_bf16x8(bh), o[db], 0, 0, 0);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[db]), as_bf16x8(bl), o[db], 0, 0, 0);
      }
    }
  };

  // ---- the key tiles ------------------------------------------------------------------------------
  fetch_idx(0, ik_n, iv_n, ok_n);
  if constexpr (QL) {
    // tile k + 1's keys and values load while tile k is consumed
    // two LDS buffers: tile k + 1 is stored, and tile k + 2 loaded into registers, while tile k
    // is consumed; one barrier per tile
    fetch(0, ik_n, iv_n, ok_n);
    if (1 < n_tiles) fetch_idx(1, ik_n, iv_n, ok_n);
    store(0);
    if (1 < n_tiles) {
      fetch(1, ik_n, iv_n, ok_n);
      if (2 < n_tiles) fetch_idx(2, ik_n, iv_n, ok_n);
    }
    for (int k = 0; k < n_tiles; ++k) {
      __syncthreads();                // tile k is staged; every wave is done with tile k - 1
      ks = ks2[k & 1];
      vt = vt2[k & 1];
      const Tile tl = tile_of(k);
      consume(tl.count, tl.seg == 3 ? tl.start : -1);
      // tile k + 1 is staged after the products of tile k are issued, so the staging work runs
      // while they drain (its buffer last served tile k - 1, which the barrier above closed)
      if (k + 1 < n_tiles) {
        ks = ks2[(k + 1) & 1];
        vt = vt2[(k + 1) & 1];
        store(k + 1);
        if (k + 2 < n_tiles) {
          fetch(k + 2, ik_n, iv_n, ok_n);
          if (k + 3 < n_tiles) fetch_idx(k + 3, ik_n, iv_n, ok_n);
        }
      }
    }
  } else {
    for (int k = 0; k < n_tiles; ++k) {
      fetch(k, ik_n, iv_n, ok_n);
      if (k + 1 < n_tiles) fetch_idx(k + 1, ik_n, iv_n, ok_n);
      __syncthreads();                // every wave is done with the previous tile
      store(k);
      __syncthreads();
      const Tile tl = tile_of(k);
      consume(tl.count, tl.seg == 3 ? tl.start : -1);
    }
  }

  // ---- normalise and write: O^T register r of block db is channel 32db + 8(r/4) + 4half + r%4
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (active) {
    const float inv = 1.f / l_tot;
    float* orow = p.out + (((int64_t)b * p.M + qi) * p.Hq + hq) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const float4 v = {o[db][4 * r4] * inv, o[db][4 * r4 + 1] * inv, o[db][4 * r4 + 2] * inv,
                          o[db][4 * r4 + 3] * inv};
        *reinterpret_cast<float4*>(orow + 32 * db + 8 * r4 + 4 * half) = v;
      }
  }
}

}  // namespace

template <int NG, int C>
hipError_t launch_extend_variant(const ExtendParams& p, hipStream_t stream) {
  const dim3 grid((unsigned)((int64_t)p.B * p.Hkv * p.row_blocks));
  if (p.rot)
    hipLaunchKernelGGL((extend_kernel<NG, C, true>), grid, dim3(256), 0, stream, p);   // 128 rows
  else
    hipLaunchKernelGGL((extend_kernel<NG, C, false>), grid, dim3(512), 0, stream, p);  // 256 rows
  return hipGetLastError();
}

hipError_t launch_extend(const ExtendParams& p, int ng, int c, hipStream_t stream) {
  if (ng == 32 && c == 4) return launch_extend_variant<32, 4>(p, stream);
  if (ng == 16 && c == 4) return launch_extend_variant<16, 4>(p, stream);
  if (ng == 16 && c == 8) return launch_extend_variant<16, 8>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace lvq
