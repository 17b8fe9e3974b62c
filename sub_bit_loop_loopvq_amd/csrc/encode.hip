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
//    the range at a time and up to 8 tiles of 32 rows.  The host picks the group range:
//    small batches (tokens leaving the recent window) spread groups over workgroups,
//    bulk encodes give a workgroup all groups of its rows so whole cache rows are read.
//  * screen: D_k = ||C_k||^2 + ||x||^2 - 2 x.C_k for a 32-codeword x 32-row tile is two
//    bf16 32x32x16 MFMAs: the first seeds the accumulator with the two squared norms
//    (each split exactly into three bf16 parts), the second adds C . (-2x) (the -2 is
//    exact in bf16).  Each lane holds 128 of its row's 256 distances.
//  * epilogue: each distance is packed with its codeword index in the low 8 mantissa
//    bits; a running min and med3 keep the two smallest packed keys (3 VALU ops per
//    distance).  The two half-waves that share a row are merged.
//  * exactness: the screen errs by at most delta = 2^-16 (||x||^2 + max_k ||C_k||^2)
//    and the packing truncates by at most 2^-15 relative.  If the two smallest keys
//    are further apart than both bounds allow, the screened winner is the exact
//    argmin.  Otherwise the row's tile is screened again and every codeword within the
//    bound of the minimum is re-scored as a sequential fp64 sum of squared
//    differences; the lowest exact minimiser wins (the brute-force definition).
//  * packing: the 8-bit index is stored as one byte of its 16-index micro-tile
//    (token quad x group quad) in the page the block table maps its position to.
#include "lvq_common.h"

namespace lvq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));


__device__ __forceinline__ uint32_t neg2_bf16x2(uint32_t w) {
  // -2 * (two packed bf16); exact: doubling only changes the exponent
  const float lo = -2.0f * __uint_as_float(w << 16);
  const float hi = -2.0f * __uint_as_float(w & 0xffff0000u);
  return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xffff0000u);
}

// v -> (hi, mid, lo) bf16 parts with hi + mid + lo == v to within 2^-24 |v| (truncating splits)
__device__ __forceinline__ void split3(float v, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
  const uint32_t b0 = __float_as_uint(v) & 0xffff0000u;
  const float r1 = v - __uint_as_float(b0);
  const uint32_t b1 = __float_as_uint(r1) & 0xffff0000u;
  const float r2 = r1 - __uint_as_float(b1);
  const uint32_t b2 = __float_as_uint(r2) & 0xffff0000u;
  hi = b0 >> 16;
  mid = b1 >> 16;
  lo = b2 >> 16;
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

template <int C, int TT>
__global__ void __launch_bounds__(256) encode_kernel(EncodeParams p, int groups_per_wg) {
  constexpr int E = 4 * C;        // sub-vector length (G = 4 loop steps)
  constexpr int NMF = E / 16;     // code MFMAs per distance tile

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5, col = lane & 31;
  const int g0 = blockIdx.x * groups_per_wg;
  const int row0 = blockIdx.y * (32 * TT);
  const int h = blockIdx.z;
  const int NG = p.NG;

  const uint16_t* cb_h = p.cb_lj + (int64_t)h * NG * kCodes * E;
  const float* nrm_h = p.norms_lj + (int64_t)h * NG * kCodes;
  uint8_t* pool_h = p.pool_lj + (int64_t)h * p.head_stride;
  const int pt_mask = (1 << p.pt_shift) - 1;
  const uint32_t one2 = 0x3f803f80u;   // two bf16 ones
  __shared__ u32x4 xrow[4][32][E / 8];  // exact re-rank: the 32 sub-vectors of one tile per wave

  for (int g = g0 + wave; g < g0 + groups_per_wg && g < NG; g += 4) {
    const uint16_t* cb_g = cb_h + (int64_t)g * kCodes * E;
    const float* nrm_g = nrm_h + g * kCodes;

    // ---- rows of this pass: raw sub-vector elements [16m + 8*half, +8) of row col ----
    u32x4 xb[TT][NMF];             // -2x, the B operand of the code MFMAs
    u32x4 bn[TT];                  // B operand of the norm MFMA: [1, 1, 1, |x|^2 parts, 0, 0]
    float xn[TT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      const int r = row0 + tt * 32 + col;
      const bool ok = r < p.n_tokens;
      const uint16_t* base = p.src + (int64_t)r * p.stride_token + (int64_t)h * p.stride_head;
      float nn = 0.f;
#pragma unroll
      for (int m = 0; m < NMF; ++m) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (ok) {
          if constexpr (C == 4) {
            const int t0 = 2 * half;      // elements 8*half .. +7 = loop steps 2*half, 2*half+1
            const uint2 lo = *reinterpret_cast<const uint2*>(base + t0 * p.stride_loop + g * 4);
            const uint2 hi = *reinterpret_cast<const uint2*>(base + (t0 + 1) * p.stride_loop + g * 4);
            v = u32x4{lo.x, lo.y, hi.x, hi.y};
          } else {
            const int t0 = 2 * m + half;  // elements 16m + 8*half .. +7 = loop step 2m + half
            v = *reinterpret_cast<const u32x4*>(base + t0 * p.stride_loop + g * 8);
          }
        }
        xb[tt][m] = u32x4{neg2_bf16x2(v[0]), neg2_bf16x2(v[1]), neg2_bf16x2(v[2]), neg2_bf16x2(v[3])};
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float a = bf16_lo(v[w]), b = bf16_hi(v[w]);
          nn = fmaf(a, a, nn);
          nn = fmaf(b, b, nn);
        }
      }
      nn += __shfl_xor(nn, 32, 64);
      xn[tt] = nn;
      uint32_t xh, xm, xl;
      split3(nn, xh, xm, xl);
      bn[tt] = half == 0 ? u32x4{one2, 0x3f80u | (xh << 16), xm | (xl << 16), 0u} : u32x4{0u, 0u, 0u, 0u};
    }

    // largest squared codeword norm of this group (for the screen's error bound)
    float cmax = fmaxf(fmaxf(nrm_g[lane], nrm_g[lane + 64]), fmaxf(nrm_g[lane + 128], nrm_g[lane + 192]));
    cmax = wave_max(cmax);

    auto load_code = [&](int ct, u32x4* a, u32x4& an) {
#pragma unroll
      for (int m = 0; m < NMF; ++m)
        a[m] = *reinterpret_cast<const u32x4*>(cb_g + (ct * 32 + col) * E + 16 * m + 8 * half);
      uint32_t nh, nm, nl;
      split3(nrm_g[ct * 32 + col], nh, nm, nl);
      an = half == 0 ? u32x4{nh | (nm << 16), nl | (0x3f80u << 16), one2, 0u} : u32x4{0u, 0u, 0u, 0u};
    };
    auto screen = [&](const u32x4* a, const u32x4& an, int tt) -> f32x16 {
      f32x16 acc = {};
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(an), as_bf16x8(bn[tt]), acc, 0, 0, 0);
#pragma unroll
      for (int m = 0; m < NMF; ++m)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[m]), as_bf16x8(xb[tt][m]), acc, 0, 0, 0);
      return acc;
    };

    // ---- screen: 8 tiles of 32 codewords; keep the two smallest packed keys per lane ----
    // key = distance bits with the low 8 mantissa bits replaced by the index within the
    // lane's codeword set (k = local + 4 * half)
    float b1[TT], b2[TT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      b1[tt] = INFINITY;
      b2[tt] = INFINITY;
    }
    u32x4 a_cur[NMF], an_cur;
    load_code(0, a_cur, an_cur);
#pragma unroll 1
    for (int ct = 0; ct < kCodes / 32; ++ct) {
      u32x4 a_nxt[NMF], an_nxt;
      load_code(ct + 1 < kCodes / 32 ? ct + 1 : ct, a_nxt, an_nxt);
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        const f32x16 acc = screen(a_cur, an_cur, tt);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const uint32_t kl = (uint32_t)(ct * 32 + 8 * (r >> 2) + (r & 3));
          const float key = __uint_as_float((__float_as_uint(acc[r]) & 0xffffff00u) | kl);
          const float ob1 = b1[tt];
          b1[tt] = fminf(ob1, key);
          b2[tt] = __builtin_amdgcn_fmed3f(ob1, b2[tt], key);
        }
      }
#pragma unroll
      for (int m = 0; m < NMF; ++m) a_cur[m] = a_nxt[m];
      an_cur = an_nxt;
    }

    // ---- merge the two half-waves and decide ----
    uint32_t best[TT];
    bool rerank[TT];
    float thr[TT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      const bool ok = row0 + tt * 32 + col < p.n_tokens;
      // the lane's own keys carry local indices; make them global (k = local + 4*half)
      const float ob1 = __shfl_xor(b1[tt], 32, 64);
      const float ob2 = __shfl_xor(b2[tt], 32, 64);
      const uint32_t myk = (__float_as_uint(b1[tt]) & 0xffu) + 4u * half;
      const uint32_t ok1 = (__float_as_uint(ob1) & 0xffu) + 4u * (half ^ 1);
      const float v1 = __uint_as_float(__float_as_uint(b1[tt]) & 0xffffff00u);
      const float w1 = __uint_as_float(__float_as_uint(ob1) & 0xffffff00u);
      float nb1, nb2;
      uint32_t nk1;
      if (w1 < v1 || (w1 == v1 && ok1 < myk)) {
        nb1 = w1;
        nk1 = ok1;
        nb2 = fminf(v1, __uint_as_float(__float_as_uint(ob2) & 0xffffff00u));
      } else {
        nb1 = v1;
        nk1 = myk;
        nb2 = fminf(__uint_as_float(__float_as_uint(b2[tt]) & 0xffffff00u), w1);
      }
      const float delta = 1.52587890625e-05f * (xn[tt] + cmax);              // 2^-16 (|x|^2 + max|C|^2)
      const float trunc = 6.103515625e-05f * fmaxf(fabsf(nb1), fabsf(nb2));   // 2^-14 max(|b1|, |b2|)
      rerank[tt] = ok && !(nb2 - nb1 > 2.f * delta + trunc);
      thr[tt] = nb1 + 6.103515625e-05f * fabsf(nb1) + 2.f * delta + trunc;
      best[tt] = nk1;
    }

    // ---- rare: exact re-rank.  The tile is screened again and every codeword whose screened
    //      distance is within the bound of the minimum is re-scored in fp64 (sequential over
    //      elements, no fused operations); the lowest exact minimiser wins. ----
    bool any_rr = false;
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) any_rr |= rerank[tt];
    if (__any(any_rr)) {
#pragma unroll 1
      for (int ts = 0; ts < TT; ++ts) {
        // the selected tile's operands, picked with uniform selects (no dynamic register indexing)
        u32x4 xs[NMF], bs = bn[0];
        bool rs = rerank[0];
        float ts_thr = thr[0];
#pragma unroll
        for (int m = 0; m < NMF; ++m) xs[m] = xb[0][m];
#pragma unroll
        for (int tt = 1; tt < TT; ++tt) {
          if (ts == tt) {
#pragma unroll
            for (int m = 0; m < NMF; ++m) xs[m] = xb[tt][m];
            bs = bn[tt];
            rs = rerank[tt];
            ts_thr = thr[tt];
          }
        }
        if (!__any(rs)) continue;
        // park the rows (x = -0.5 * (-2x), exact) in LDS for the fp64 pass
#pragma unroll
        for (int m = 0; m < NMF; ++m) {
          u32x4 xw;
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const uint32_t nw = xs[m][w];
            const float lo = -0.5f * bf16_lo(nw), hi = -0.5f * bf16_hi(nw);
            xw[w] = (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xffff0000u);
          }
          xrow[wave][col][2 * m + half] = xw;
        }
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        double bd = INFINITY;
        uint32_t bk = 0xffffffffu;
#pragma unroll 1
        for (int ct = 0; ct < kCodes / 32; ++ct) {
          u32x4 a[NMF], an;
          load_code(ct, a, an);
          f32x16 acc = {};
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(an), as_bf16x8(bs), acc, 0, 0, 0);
#pragma unroll
          for (int m = 0; m < NMF; ++m)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[m]), as_bf16x8(xs[m]), acc, 0, 0, 0);
          uint32_t mask = 0u;
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) mask |= (acc[rr] <= ts_thr ? 1u : 0u) << rr;
          if (!rs) mask = 0u;
          while (mask) {                      // candidates of this lane (rare, divergent)
            const int rr = __builtin_ctz(mask);
            mask &= mask - 1u;
            const uint32_t k = (uint32_t)(ct * 32 + 8 * (rr >> 2) + 4 * half + (rr & 3));
            const u32x4* ck = reinterpret_cast<const u32x4*>(cb_g + k * E);
            double dd = 0.0;
#pragma unroll 1
            for (int e8 = 0; e8 < E / 8; ++e8) {
              const u32x4 xv = xrow[wave][col][e8];
              const u32x4 cv = ck[e8];
#pragma unroll
              for (int w = 0; w < 4; ++w) {
                const double d0 = __dsub_rn((double)bf16_lo(xv[w]), (double)bf16_lo(cv[w]));
                dd = __dadd_rn(dd, __dmul_rn(d0, d0));
                const double d1 = __dsub_rn((double)bf16_hi(xv[w]), (double)bf16_hi(cv[w]));
                dd = __dadd_rn(dd, __dmul_rn(d1, d1));
              }
            }
            if (dd < bd || (dd == bd && k < bk)) {
              bd = dd;
              bk = k;
            }
          }
        }
        // merge the two halves' exact candidates (lowest index on equal distance)
        const double obd = __shfl_xor(bd, 32, 64);
        const uint32_t obk = __shfl_xor(bk, 32, 64);
        if (obd < bd || (obd == bd && obk < bk)) bk = obk;
        if (rs && p.rerank_count && half == 0) atomicAdd(p.rerank_count, 1ull);
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
          if (ts == tt && rs) best[tt] = bk;
        __builtin_amdgcn_wave_barrier();
      }
    }

    // ---- store ----
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      const int r = row0 + tt * 32 + col;
      if (half == 0 && r < p.n_tokens) {
        if (p.out_idx) p.out_idx[((int64_t)r * p.Hkv + h) * NG + g] = (int)best[tt];
        const int seq = p.seq_id[r];
        const int u = p.vq_pos[r];
        if (seq >= 0 && seq < p.batch && u >= 0 && (u >> p.pt_shift) < p.max_pages) {
          const int page = p.block_table[(int64_t)seq * p.max_pages + (u >> p.pt_shift)];
          if (page >= 0 && page < p.num_pages) {
            const int w = u & pt_mask;
            const int64_t off = (int64_t)page * p.page_bytes + (int64_t)p.kind * p.kind_bytes +
                                ((w >> 2) * (NG >> 2) + (g >> 2)) * 16 + (w & 3) * 4 + (g & 3);
            pool_h[off] = (uint8_t)best[tt];
          }
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_encode(const EncodeParams& p, int c, hipStream_t stream) {
  if (p.n_tokens == 0) return hipSuccess;
  // small batches (tokens leaving the recent window): one group per wave, spread over many
  // workgroups; bulk: a workgroup owns every group of 128 rows, so each cache row is read
  // whole by one workgroup
  const bool small = (int64_t)p.n_tokens * p.Hkv < 16384;
  const int groups_per_wg = small ? 4 : p.NG;
  const int rows_per_wg = small ? 64 : 128;
  const dim3 grid((p.NG + groups_per_wg - 1) / groups_per_wg, (p.n_tokens + rows_per_wg - 1) / rows_per_wg, p.Hkv);
  if (c == 4 && small)
    hipLaunchKernelGGL((encode_kernel<4, 2>), grid, dim3(256), 0, stream, p, groups_per_wg);
  else if (c == 4)
    hipLaunchKernelGGL((encode_kernel<4, 4>), grid, dim3(256), 0, stream, p, groups_per_wg);
  else if (c == 8 && small)
    hipLaunchKernelGGL((encode_kernel<8, 2>), grid, dim3(256), 0, stream, p, groups_per_wg);
  else if (c == 8)
    hipLaunchKernelGGL((encode_kernel<8, 4>), grid, dim3(256), 0, stream, p, groups_per_wg);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace lvq
