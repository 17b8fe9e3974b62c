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
//  * workgroup = 256 query rows (row = (chunk token, q-head of the kv-head)) of one
//    (sequence, kv-head); 8 waves of 32 rows, one workgroup per CU.  Keys come in tiles of 64
//    tokens, staged in LDS by the whole workgroup into two buffers (tile k + 1 while tile k is
//    consumed): K as [token][d] bf16 rows (padded so the MFMA operand reads hit distinct banks)
//    and V as [token][d] rows too, whose 16-byte chunks are XOR-permuted per row; the value
//    product reads its V^T operand with the transposing LDS read (ds_read_b64_tr_b16), so
//    staging writes whole 16-byte chunks.  Vector-quantized tokens are dequantized on the
//    way: the packed index byte of (token, group) selects the c channels of that group's
//    loop-step slice; keys from the kv-head's key slice, copied to LDS once, values from the
//    group-major codebook copy ([tau][g][k][i]) in L2.
//  * per wave: S^T = K Q^T on bf16 32x32x16 MFMAs (a rotated q' = R^T q is split into two
//    bf16 parts, two MFMAs), online softmax in log2 units with the causal mask of the chunk,
//    then O^T += V^T P^T: on fp16 MFMAs with P rounded to fp16 while every value converts to
//    fp16 exactly, else with P split into two bf16 parts (hi + lo, 2^-16 relative).  The
//    D-layout of S^T (lane = query row, registers = tokens) is directly the B operand of the
//    second product once its 16 tokens are taken in the order the registers hold them; the
//    transposing reads gather the V^T operand in the same order.
#include "lvq_common.h"

namespace lvq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kKT = 64;        // keys per tile
// s_waitcnt immediate (gfx9 encoding): vector-memory count 0, the export and LDS/scalar counts
// left at their maxima (no wait on them)
constexpr int kWaitVmem0 = 0x0F70;
// V tiles are row-major [key][d] with the 16-byte chunks of key row t XOR-permuted by vswz(t), so
// that the 16-byte row writes of the staging (consecutive keys, one chunk) hit distinct banks.
// (The transposing operand reads keep 2-way conflicts with it; a permutation measured free of
// conflicts in both was no faster.)
__device__ __forceinline__ int vswz(int t) { return ((t & 3) << 1) | ((t >> 2) & 1); }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ f16x8 as_f16x8(u32x4 v) { return __builtin_bit_cast(f16x8, v); }

// two fp32 -> packed fp16, round to nearest even
__device__ __forceinline__ uint32_t f16x2_rne(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, f16x2));
}
// two packed bf16 -> packed fp16 (exact inside the window below)
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) { return f16x2_rne(bf16_lo(w), bf16_hi(w)); }
// The fp16 window: a bf16 value converts to fp16 exactly when it is zero or its magnitude lies in
// [2^-17, 2^16) (8 significant bits need an exponent of at least -17 in fp16, whose subnormals
// reach 2^-24; 2^16 overflows).  Magnitude bits of bf16 compare like the magnitudes; bf16
// infinities and NaNs lie above kF16Hi.
constexpr uint32_t kF16Hi = (127u + 16u) << 7;    // 2^16
constexpr uint32_t kF16Lo = (127u - 17u) << 7;    // 2^-17
// running packed statistics of the magnitude bits m of two bf16: the maximum, and the minimum
// of m - 1 (wrapping, so zeros count as 0xffff and never as small)
__device__ __forceinline__ void mag_stats(uint32_t& mx, uint32_t& mn1, uint32_t w) {
  const u16x2 m = __builtin_bit_cast(u16x2, w & 0x7fff7fffu);
  mx = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, mx), m));
  mn1 = __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(u16x2, mn1), m - (unsigned short)1));
}

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
__global__ void __launch_bounds__(512, 1) extend_kernel(ExtendParams p) {
  // 8 waves (256 query rows) per workgroup, one workgroup per CU, so that each staged tile
  // serves 256 rows.
  constexpr int NTH = 512;
  constexpr int kRows = NTH / 2;
  constexpr int D = NG * C;
  constexpr int KROW = D + 8;         // bf16 per K row (16 B of padding)
  constexpr int KSTEPS = D / 16;      // k-steps of S^T = K Q^T
  constexpr int DB = D / 32;          // 32-channel blocks of O^T
  // Two K / V^T tile buffers (tile k + 1 is staged while tile k is consumed) and the key
  // codebook's loop-step slice of the kv-head in LDS (its K x d bf16, loaded once), so that the
  // dequantization of vector-quantized keys gathers from LDS instead of L2; q stays in registers.
  __shared__ __align__(16) uint16_t ks2[2][kKT * KROW];
  __shared__ __align__(16) uint16_t vt2[2][kKT * D];
  __shared__ __align__(16) uint16_t cbk_l[kCodes * D];
  // The value tiles are staged as fp16 and the value product runs on fp16 MFMAs with P rounded
  // to fp16: one product instead of the bf16 hi + lo pair.  The first tile with a value outside
  // the fp16 window ends that loop; a second loop, in bf16, goes on from it.
  constexpr int NWAVE = NTH / 64;
  __shared__ uint32_t vbad[2][NWAVE];   // per buffer and wave: a value outside the fp16 window
  __shared__ uint32_t vslice_bad[NWAVE];   // per wave: a value of the value codebook slice outside it
  uint16_t* ks = ks2[0];
  uint16_t* vt = vt2[0];

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
  // the wave's first and last chunk tokens: a chunk tile that starts after the last is hidden from
  // all its rows, one that ends at or before the first is visible to all of them
  const int wave_last_qi = min(Mb - 1, (row_ws + wave * 32 + 31) / grp);
  const int wave_first_qi = (row_ws + wave * 32) / grp;
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
      bq[kk] = *reinterpret_cast<const u32x4*>(qrow + 16 * kk + 8 * half);
      bq_lo[kk] = u32x4{0u, 0u, 0u, 0u};
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
  // chunk's tiles up to the workgroup's last row.  While tile k is consumed, tile k + 1 is written
  // to the other LDS buffer and the loads of the tiles after it are in flight (see the loop).
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
  // vector-quantized items: (token, GPI consecutive groups inside one group quad), as many as
  // there are threads when the quads allow it (fewer staging registers per thread at c = 8)
  constexpr int GPI = NG * kKT / NTH >= 4 ? 4 : (NG * kKT / NTH >= 2 ? 2 : 1);
  constexpr int QIT = kKT * (NG / GPI);             // items of a tile
  constexpr int QITEMS = (QIT + NTH - 1) / NTH;     // per thread (the last may be idle)
  constexpr bool kAllLive = QIT % NTH == 0;
  static_assert(RITEMS >= 1 && RITEMS * NTH == kKT * PIECES && QITEMS >= 1, "tile mapping");
  constexpr int FB = RITEMS * 4 > QITEMS * GPI * (C / 2) ? RITEMS * 4 : QITEMS * GPI * (C / 2);   // dwords per kind
  uint32_t fk[FB], fv[FB];          // the tile's keys / values on their way to LDS
  uint32_t ik_n[QITEMS], iv_n[QITEMS];   // packed indices of the next tile
  bool ok_n[QITEMS];

  // Packed indices of vector-quantized tiles.  Tile k's page id, then its index dwords, then its
  // codewords are three dependent loads; each is requested a tile before the next needs it, and
  // all three kinds are read at valid addresses for every tile ordinal (an ordinal outside the
  // vector-quantized tiles reads a clamped one, marked not ok), so every tile issues the same
  // loads.  Loads complete in issue order: a tile's waits all come before its new requests, so
  // that a wait never covers a load issued in the same tile step.
  const bool has_vq = t_vq > 0;    // (uniform) pool and block table are read only then
  auto vq_tile = [&](int k) -> Tile {
    const int j = min(max(k - t_pre, 0), t_vq - 1);
    return {1, j * kKT, n_vq - j * kKT};
  };
  // the page of tile k (the tile is 64 aligned positions and a page holds a power of two >= 64, so
  // one page per tile).  The offset carries a zero the compiler cannot see as uniform, so the id
  // stays in a vector register until it is used instead of being moved to a scalar register, and
  // waited for, at once.
  auto fetch_page = [&](int k) -> int {
    int vz;
    asm("v_mov_b32 %0, 0" : "=v"(vz));
    return p.block_table[(int64_t)b * p.max_pages + (vq_tile(k).start >> p.pt_shift) + vz];
  };
  // addresses of tile k's index dwords in its page (token quads x group quads), with ok flags
  struct IdxPlan {
    const uint8_t* at[QITEMS];
    bool ok[QITEMS];
  };
  auto plan_idx = [&](int k, int page) -> IdxPlan {
    const bool real = k < n_tiles && tile_of(k).seg == 1;
    const Tile tl = vq_tile(k);
    const bool pok = page >= 0 && page < p.num_pages;
    page = pok ? page : 0;
    IdxPlan ip;
#pragma unroll
    for (int m = 0; m < QITEMS; ++m) {
      const int it0 = tid + NTH * m;
      const bool live = kAllLive || it0 < QIT;
      const int it = live ? it0 : 0;
      const int t = it % kKT, gq = (it / kKT) * GPI / 4;   // the item's group quad
      ip.ok[m] = real && live && pok && t < tl.count;
      const int w = (tl.start + min(t, tl.count - 1)) & pt_mask;
      ip.at[m] = pool_h + (int64_t)page * p.page_bytes + (((w >> 2) * (NG / 4) + gq) * 16 + (w & 3) * 4);
    }
    return ip;
  };
  auto issue_idx = [&](const IdxPlan& ip, uint32_t* ik, uint32_t* iv, bool* ok) {
#pragma unroll
    for (int m = 0; m < QITEMS; ++m) {
      ik[m] = *reinterpret_cast<const uint32_t*>(ip.at[m]);
      iv[m] = *reinterpret_cast<const uint32_t*>(ip.at[m] + p.kind_bytes);
      ok[m] = ip.ok[m];
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
        const int g0 = GPI * ((kAllLive || it0 < QIT ? it0 : 0) / kKT);   // first group of the item
#pragma unroll
        for (int r = 0; r < GPI; ++r) {
          const int g = g0 + r, sh = 8 * (g & 3);   // index byte g % 4 of the quad's dword
          const uint32_t kx = (ik[m] >> sh) & 0xffu, vx = (iv[m] >> sh) & 0xffu;
          const uint32_t* kc = reinterpret_cast<const uint32_t*>(cbk_l + (g * kCodes + kx) * C);
          const uint32_t* vc = reinterpret_cast<const uint32_t*>(slice_v + (g * kCodes + vx) * C);
#pragma unroll
          for (int e = 0; e < C / 2; ++e) {
            fk[(m * GPI + r) * (C / 2) + e] = kc[e];
            fv[(m * GPI + r) * (C / 2) + e] = vc[e];
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
  // the registers of tile k into LDS: K and V as [token][d] (V chunks permuted by vswz); entries
  // past the tile's keys are written as zeros
  // (values as fp16 when the tag is true, with the wave's window flag for buffer par)
  auto store = [&](int k, int par, auto as_f16) {
    constexpr bool AS = decltype(as_f16)::value;
    const Tile tl = tile_of(k);
    uint32_t mx = 0u, mn1 = 0xffffffffu;
    // (vector-quantized values come from the codebook slice, checked once per workgroup)
    auto vconv = [&](uint32_t w, auto chk) -> uint32_t {
      if constexpr (AS) {
        if constexpr (decltype(chk)::value) mag_stats(mx, mn1, w);
        return bf16x2_to_f16x2(w);
      } else {
        return w;
      }
    };
    if (tl.seg == 1) {
#pragma unroll
      for (int m = 0; m < QITEMS; ++m) {
        const int it = tid + NTH * m;
        if (!kAllLive && it >= QIT) continue;
        const int t = it % kKT, g0 = GPI * (it / kKT);
        const uint32_t keep = ok_cur[m] ? 0xffffffffu : 0u;
#pragma unroll
        for (int r = 0; r < GPI; ++r) {
          uint32_t* kd = reinterpret_cast<uint32_t*>(ks + t * KROW + (g0 + r) * C);
#pragma unroll
          for (int e = 0; e < C / 2; ++e) kd[e] = fk[(m * GPI + r) * (C / 2) + e] & keep;
        }
        // the item's GPI * C value channels are whole 16-byte chunks of the key's V row
        constexpr int NCH = GPI * C / 8;
        static_assert(NCH * 8 == GPI * C, "value chunks");
        const int c0 = g0 * C / 8;
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
          u32x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = vconv(fv[m * GPI * (C / 2) + 4 * j + e] & keep, std::false_type{});
          *reinterpret_cast<u32x4*>(vt + t * D + 8 * ((c0 + j) ^ vswz(t))) = w;
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
        u32x4 vw;
#pragma unroll
        for (int w = 0; w < 4; ++w) vw[w] = vconv(fv[4 * m + w] & keep, std::true_type{});
        *reinterpret_cast<u32x4*>(vt + t * D + 8 * (pc ^ vswz(t))) = vw;
      }
    }
    if constexpr (AS) {
      const uint32_t top = max(mx >> 16, mx & 0xffffu), bot = min(mn1 >> 16, mn1 & 0xffffu);
      const bool out = top >= kF16Hi || bot < kF16Lo - 1u;
      const bool bad = __builtin_amdgcn_ballot_w64(out) != 0;
      if (lane == 0) vbad[par][wave] = bad ? 1u : 0u;
    }
  };

  // ---- one staged tile: scores, online softmax, value products --------------------------------
  // chunk_j0 >= 0 marks chunk keys: key t is chunk token chunk_j0 + t (causal); count = valid keys.
  // Rows past the chunk length compute on row 0's q and are never written, so they need no mask.
  // The softmax reference m_ref (log2 units) moves only when a score exceeds it by more than
  // 8: exponentials stay <= 2^8 and o, l are rescaled rarely.
  const float cl2 = p.scale_log2;
  auto consume = [&](int count, int chunk_j0, auto f16) {
    // (with a rotation the lane's operand addresses are recomputed from a fresh lane id in every
    // tile, so that they are not kept live, or spilled, across the tile loop)
    int lane_f = lane;
    if constexpr (ROT) asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane_f));
    const int col = lane_f & 31, half = lane_f >> 5;
    // transposing V reads: key row 4 half + s/4 of a k-step's 8-key half, logical chunk
    // 4 db + 2 (lane / 16 % 2) + (s % 4) / 2, XOR-permuted by vswz of the row (= 2 (s/4) + half)
    const int vs = lane_f & 15;
    const int vkl = (2 * ((lane_f >> 4) & 1) + ((vs & 3) >> 1)) ^ (2 * (vs >> 2) + half);
    const int vlane = (4 * half + (vs >> 2)) * 2 * D + 8 * (vs & 1);
    // NB 32-key blocks per pass: without a rotation both blocks of the tile in one pass; with one
    // (q' in two parts takes 32 more registers), one block per pass, so that the scores and the
    // key operands of only half the tile are live at once.
    constexpr int NB = ROT ? 1 : 2;
    constexpr int KB = ROT ? KSTEPS / 2 : KSTEPS;   // key operands loaded together
    float psum = 0.f;
#pragma unroll
    for (int pass = 0; pass < 2 / NB; ++pass) {
      f32x16 s[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int mb = pass * NB + b;
        const uint16_t* krow = ks + (32 * mb + col) * KROW + 8 * half;
        f32x16 acc = {};
#pragma unroll
        for (int k0 = 0; k0 < KSTEPS; k0 += KB) {
          // KB of the block's K operands first, so the LDS reads overlap instead of each MFMA
          // waiting for its own
          u32x4 a[KB];
#pragma unroll
          for (int kk = 0; kk < KB; ++kk) a[kk] = *reinterpret_cast<const u32x4*>(krow + 16 * (k0 + kk));
#pragma unroll
          for (int kk = 0; kk < KB; ++kk) {
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[kk]), as_bf16x8(bq[k0 + kk]), acc, 0, 0, 0);
            if constexpr (ROT)
              acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[kk]), as_bf16x8(bq_lo[k0 + kk]), acc, 0, 0, 0);
          }
        }
        s[b] = acc;
      }
      // raw scores; token of register r of block mb: 32mb + 8(r/4) + 4half + r%4
      if (count < kKT || (chunk_j0 >= 0 && chunk_j0 + kKT - 1 > wave_first_qi)) {   // (uniform) keys to hide
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int t = 32 * (pass * NB + b) + 8 * (r >> 2) + 4 * half + (r & 3);
            const bool vis = t < count && (chunk_j0 < 0 || chunk_j0 + t <= qi);
            s[b][r] = vis ? s[b][r] : -INFINITY;
          }
      }
      float tmax = -INFINITY;
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, s[b][r]);
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64)) * cl2;
      const bool move = tmax > m_ref + 8.f;       // m_ref = -inf: any visible key moves it
      if (__builtin_amdgcn_ballot_w64(move)) {
        const float alpha = move ? __builtin_amdgcn_exp2f(m_ref - tmax) : 1.f;   // m_ref = -inf -> 0
        m_ref = move ? tmax : m_ref;
        l_run *= alpha;
        psum *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
      }
      // (a row with nothing visible yet keeps m_ref = -inf and uses 0, so exp2(-inf) = 0)
      const float nm = m_ref == -INFINITY ? 0.f : -m_ref;
      // l: the sum of the weights the value product uses (fp16 tiles: of the rounded ones, added
      // pairwise by v_dot2_f32_f16 while they are packed)
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = __builtin_amdgcn_exp2f(fmaf(s[b][r], cl2, nm));
          s[b][r] = e;
          if constexpr (!decltype(f16)::value) psum += e;
        }
      // O^T += V^T P^T over the pass's k-steps of 16 keys.  fp16 tiles: P rounded to nearest fp16
      // (2^-11 relative, 2^-25 absolute below 2^-14), one product.  bf16 tiles: P = hi + lo with
      // hi the truncated upper half and lo = P - hi (exact) rounded to bf16 by the hardware
      // conversion, 2^-16 relative, two products.
#pragma unroll
      for (int ks2i = 0; ks2i < 2 * NB; ++ks2i) {
        const int kst = 2 * NB * pass + ks2i, b = ks2i >> 1, r0 = 8 * (ks2i & 1);
        // V^T operand by transposing reads: lane s of each 16 points at 4 channels of key row
        // 16 kst + 8 rd + 4 half + s/4, and receives its own channel of those 4 keys
        u32x4 a[DB];
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const uint8_t* vb = reinterpret_cast<const uint8_t*>(vt) + vlane + 16 * ((4 * db) ^ vkl) + 32 * D * kst;
          const i16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vb));
          const i16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vb + 16 * D));
          const uint2 u0 = __builtin_bit_cast(uint2, r0), u1 = __builtin_bit_cast(uint2, r1);
          a[db] = u32x4{u0.x, u0.y, u1.x, u1.y};
        }
        if constexpr (decltype(f16)::value) {
          uint32_t pw[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            pw[j] = f16x2_rne(s[b][r0 + 2 * j], s[b][r0 + 2 * j + 1]);
            psum = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pw[j]), f16x2{1.0f16, 1.0f16}, psum, false);
          }
          const u32x4 bp = {pw[0], pw[1], pw[2], pw[3]};
#pragma unroll
          for (int db = 0; db < DB; ++db)
            o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_f16x8(a[db]), as_f16x8(bp), o[db], 0, 0, 0);
        } else {
          uint32_t hw[4], lw[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t ua = __float_as_uint(s[b][r0 + 2 * j]), ub = __float_as_uint(s[b][r0 + 2 * j + 1]);
            hw[j] = __builtin_amdgcn_perm(ub, ua, 0x07060302u);
            const f32x2 lo = {__uint_as_float(ua) - __uint_as_float(ua & 0xffff0000u),
                              __uint_as_float(ub) - __uint_as_float(ub & 0xffff0000u)};
            lw[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf16x2));
          }
          const u32x4 bh = {hw[0], hw[1], hw[2], hw[3]};
          const u32x4 bl = {lw[0], lw[1], lw[2], lw[3]};
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[db]), as_bf16x8(bh), o[db], 0, 0, 0);
            o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[db]), as_bf16x8(bl), o[db], 0, 0, 0);
          }
        }
      }
    }
    l_run += psum;
  };

  // whether every value of the tile in buffer par lies in the fp16 window, from the waves'
  // flags (read after the barrier that closes its staging)
  auto tile_f16 = [&](int par) -> bool {
    uint32_t f = 0u;
#pragma unroll
    for (int w = 0; w < NWAVE; ++w) f |= vbad[par][w];
    return f == 0u;
  };

  // ---- the key tiles ------------------------------------------------------------------------------
  bool vq_f16 = true;   // every value of the value codebook slice lies in the fp16 window
  if (t_vq > 0) {   // (uniform)
    constexpr int PER = kCodes * D * 2 / 16 / NTH;
    static_assert(PER * NTH * 16 == kCodes * D * 2, "codebook staging");
    // the key codebook slice into LDS, 16 B per thread and step
#pragma unroll
    for (int m = 0; m < PER; ++m)
      reinterpret_cast<u32x4*>(cbk_l)[tid + NTH * m] = reinterpret_cast<const u32x4*>(slice_k)[tid + NTH * m];
    // the value slice against the fp16 window, once
    uint32_t mx = 0u, mn1 = 0xffffffffu;
#pragma unroll
    for (int m = 0; m < PER; ++m) {
      const u32x4 w = reinterpret_cast<const u32x4*>(slice_v)[tid + NTH * m];
#pragma unroll
      for (int e = 0; e < 4; ++e) mag_stats(mx, mn1, w[e]);
    }
    const uint32_t top = max(mx >> 16, mx & 0xffffu), bot = min(mn1 >> 16, mn1 & 0xffffu);
    const bool bad = __builtin_amdgcn_ballot_w64(top >= kF16Hi || bot < kF16Lo - 1u) != 0;
    if (lane == 0) vslice_bad[wave] = bad ? 1u : 0u;
    __syncthreads();
    uint32_t f = 0u;
#pragma unroll
    for (int w = 0; w < NWAVE; ++w) f |= vslice_bad[w];
    vq_f16 = f == 0u;
  }
  // The q operand's loads are complete here on every path (the codebook staging above already
  // waited for them when it ran).  Said explicitly, so the memory-counter waits inside the tile
  // loop only cover the loop's own loads: otherwise the score products of every tile wait for all
  // loads in flight, the next tiles' gathers included.
  __builtin_amdgcn_s_waitcnt(kWaitVmem0);
  using f16_tag = std::integral_constant<bool, true>;
  using bf16_tag = std::integral_constant<bool, false>;
  {
    auto run = [&](int k0, auto tag) -> int {
      constexpr bool AS = decltype(tag)::value;
      const int last = n_tiles - 1;
      // state entering tile k: tile k in LDS, tile k + 1's keys / values requested into fk / fv,
      // tile k + 2's index dwords into ik_n / iv_n, tile k + 3's page id into pg_n
      int pg_n = 0;
      IdxPlan ip;
      if (has_vq) {
        issue_idx(plan_idx(k0, fetch_page(k0)), ik_n, iv_n, ok_n);
        pg_n = fetch_page(min(k0 + 1, last));
      }
      fetch(k0, ik_n, iv_n, ok_n);
      if (has_vq) {
        issue_idx(plan_idx(k0 + 1, pg_n), ik_n, iv_n, ok_n);
        pg_n = fetch_page(min(k0 + 2, last));
      }
      ks = ks2[k0 & 1];
      vt = vt2[k0 & 1];
      store(k0, k0 & 1, tag);
      if (k0 + 1 < n_tiles) {
        if (has_vq) ip = plan_idx(k0 + 2, pg_n);
        fetch(k0 + 1, ik_n, iv_n, ok_n);
        if (has_vq) {
          issue_idx(ip, ik_n, iv_n, ok_n);
          pg_n = fetch_page(min(k0 + 3, last));
        }
      }
      for (int k = k0; k < n_tiles; ++k) {
        __syncthreads();              // tile k is staged; every wave is done with tile k - 1
        if constexpr (AS) {
          if (!tile_f16(k & 1)) return k;   // (uniform) nobody reads tile k's buffers any more
        }
        ks = ks2[k & 1];
        vt = vt2[k & 1];
        const Tile tl = tile_of(k);
        if (tl.seg != 3 || tl.start <= wave_last_qi) consume(tl.count, tl.seg == 3 ? tl.start : -1, tag);
        // tile k + 1 is staged after the products of tile k are issued, so the staging work runs
        // while they drain (its buffer last served tile k - 1, which the barrier above closed)
        if (k + 1 < n_tiles) {
          ks = ks2[(k + 1) & 1];
          vt = vt2[(k + 1) & 1];
          store(k + 1, (k + 1) & 1, tag);
          if (k + 2 < n_tiles) {
            if (has_vq) ip = plan_idx(k + 3, pg_n);
            __builtin_amdgcn_sched_barrier(0);
            fetch(k + 2, ik_n, iv_n, ok_n);
            if (has_vq) {
              issue_idx(ip, ik_n, iv_n, ok_n);
              pg_n = fetch_page(min(k + 4, last));
            }
          }
        }
      }
      return n_tiles;
    };
    const int k0 = n_tiles > 0 && vq_f16 ? run(0, f16_tag{}) : 0;
    if (k0 < n_tiles) run(k0, bf16_tag{});
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
    // ln of the row's softmax normaliser: m_ref and l_tot are in log2 units and relative to m_ref
    // (every computed row sees at least its own chunk key, so l_tot > 0)
    if (p.lse && half == 0) p.lse[((int64_t)b * p.M + qi) * p.Hq + hq] = (m_ref + log2f(l_tot)) * 0.6931471805599453f;
  }
}

}  // namespace

template <int NG, int C>
hipError_t launch_extend_variant(const ExtendParams& p, hipStream_t stream) {
  const dim3 grid((unsigned)((int64_t)p.B * p.Hkv * p.row_blocks));
  if (p.rot)   // 256 rows per workgroup
    hipLaunchKernelGGL((extend_kernel<NG, C, true>), grid, dim3(512), 0, stream, p);
  else
    hipLaunchKernelGGL((extend_kernel<NG, C, false>), grid, dim3(512), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_extend(const ExtendParams& p, int ng, int c, hipStream_t stream) {
  if (ng == 32 && c == 4) return launch_extend_variant<32, 4>(p, stream);
  if (ng == 16 && c == 4) return launch_extend_variant<16, 4>(p, stream);
  if (ng == 16 && c == 8) return launch_extend_variant<16, 8>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace lvq
