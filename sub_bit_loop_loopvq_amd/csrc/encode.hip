// LoopVQ encode: nearest codeword of every loop-axis sub-vector, packed into index pages (gfx950).
//
// What it computes (airadar.tv summary of LoopVQ, opening summary: the channels of
// several consecutive loop steps form one sub-vector sharing one codebook index;
// section "Raisons": indices are stored packed).  For row r, kv-head h, group g the
// sub-vector x has element tau*c + i = src[tau][r][h][g*c + i]; its index is the
// lowest k minimising ||x - C_k||^2 over the K = 256 codewords of (l, h, g).
//
// How (MI355X):
//  * distances D'_k = ||C_k||^2 - 2 x.C_k are a dense contraction: a 32x32x16 bf16
//    MFMA with A = 32 codewords x E, B = E x 32 sub-vectors (pre-scaled by -2, exact
//    in bf16) and the squared norms as the accumulator input, 8 codeword tiles per
//    32 rows; each lane ends up holding 128 of its row's 256 distances.
//  * argmin epilogue per lane: best value, its index (first occurrence), and the
//    second-best value; the two half-waves that share a row are merged.
//  * exactness: the fp32 screen errs by at most
//        delta = 2^-17 * (||x||^2 + 2 max_k ||C_k||^2);
//    when the two best screened values are more than 2*delta apart the screened
//    winner is the exact argmin.  Otherwise every codeword is re-scored as a
//    sequential fp64 sum of squared differences and the lowest minimiser wins,
//    which is the brute-force definition itself.
//  * packing: the 8-bit index is stored as one byte of its 16-index micro-tile
//    (token quad x group quad) in the page the block table maps its position to.
#include "lvq_common.h"

namespace lvq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kGamma = 1.0f / 131072.0f;   // 2^-17

__device__ __forceinline__ uint32_t neg2_bf16x2(uint32_t w) {
  // -2 * (two packed bf16); exact: doubling only changes the exponent
  const float lo = -2.0f * __uint_as_float(w << 16);
  const float hi = -2.0f * __uint_as_float(w & 0xffff0000u);
  return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xffff0000u);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

template <int C>
__global__ void __launch_bounds__(256) encode_kernel(EncodeParams p) {
  constexpr int E = 4 * C;        // sub-vector length (G = 4 loop steps)
  constexpr int NMF = E / 16;     // MFMA k-steps per distance tile
  constexpr int TT = 2;           // 32-row tiles per workgroup

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5, col = lane & 31;
  const int h = blockIdx.y;
  const int row0 = blockIdx.x * (32 * TT);
  const int NG = p.NG;

  const uint16_t* cb_h = p.cb_lj + (int64_t)h * NG * kCodes * E;
  const float* nrm_h = p.norms_lj + (int64_t)h * NG * kCodes;
  uint8_t* pool_h = p.pool_lj + (int64_t)h * p.head_stride;
  const int pt_mask = (1 << p.pt_shift) - 1;

  for (int g = wave; g < NG; g += 4) {
    const uint16_t* cb_g = cb_h + (int64_t)g * kCodes * E;
    const float* nrm_g = nrm_h + g * kCodes;

    // ---- rows of this tile: raw sub-vector elements [16m + 8*half, +8) of row col ----
    u32x4 xr[TT][NMF];
    bool rvalid[TT];
    float xn[TT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      const int r = row0 + tt * 32 + col;
      rvalid[tt] = r < p.n_tokens;
      const uint16_t* base = p.src + (int64_t)r * p.stride_token + (int64_t)h * p.stride_head;
      float nn = 0.f;
#pragma unroll
      for (int m = 0; m < NMF; ++m) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (rvalid[tt]) {
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
        xr[tt][m] = v;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float a = bf16_lo(v[w]), b = bf16_hi(v[w]);
          nn = fmaf(a, a, nn);
          nn = fmaf(b, b, nn);
        }
      }
      xn[tt] = nn + __shfl_xor(nn, 32, 64);
    }
    u32x4 xb[TT][NMF];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
      for (int m = 0; m < NMF; ++m) {
        const u32x4 v = xr[tt][m];
        xb[tt][m] = u32x4{neg2_bf16x2(v[0]), neg2_bf16x2(v[1]), neg2_bf16x2(v[2]), neg2_bf16x2(v[3])};
      }

    // largest squared codeword norm of this group (for the screen's error bound)
    float cmax = fmaxf(fmaxf(nrm_g[lane], nrm_g[lane + 64]), fmaxf(nrm_g[lane + 128], nrm_g[lane + 192]));
    cmax = wave_max(cmax);

    // ---- screen: 8 tiles of 32 codewords ----
    float b1[TT], b2[TT];
    int k1[TT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      b1[tt] = INFINITY;
      b2[tt] = INFINITY;
      k1[tt] = 0;
    }
    for (int ct = 0; ct < kCodes / 32; ++ct) {
      u32x4 a[NMF];
#pragma unroll
      for (int m = 0; m < NMF; ++m)
        a[m] = *reinterpret_cast<const u32x4*>(cb_g + (ct * 32 + col) * E + 16 * m + 8 * half);
      f32x16 cin;
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const f32x4 n4 = *reinterpret_cast<const f32x4*>(nrm_g + ct * 32 + 8 * qd + 4 * half);
        cin[4 * qd + 0] = n4[0];
        cin[4 * qd + 1] = n4[1];
        cin[4 * qd + 2] = n4[2];
        cin[4 * qd + 3] = n4[3];
      }
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        f32x16 acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[0]), as_bf16x8(xb[tt][0]), cin, 0, 0, 0);
        if constexpr (NMF == 2)
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[1]), as_bf16x8(xb[tt][1]), acc, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int k = ct * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          const float v = acc[r];
          const bool lt = v < b1[tt];
          b2[tt] = lt ? b1[tt] : fminf(b2[tt], v);
          k1[tt] = lt ? k : k1[tt];
          b1[tt] = lt ? v : b1[tt];
        }
      }
    }

    // ---- merge the two half-waves, decide, re-rank if needed, store ----
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      const float ob1 = __shfl_xor(b1[tt], 32, 64);
      const float ob2 = __shfl_xor(b2[tt], 32, 64);
      const int ok1 = __shfl_xor(k1[tt], 32, 64);
      float nb1, nb2;
      int nk1;
      if (ob1 < b1[tt] || (ob1 == b1[tt] && ok1 < k1[tt])) {
        nb1 = ob1;
        nk1 = ok1;
        nb2 = fminf(b1[tt], ob2);
      } else {
        nb1 = b1[tt];
        nk1 = k1[tt];
        nb2 = fminf(b2[tt], ob1);
      }
      const float delta = kGamma * (xn[tt] + 2.f * cmax);
      const bool rerank = rvalid[tt] && !(nb2 - nb1 > 2.f * delta);
      int best = nk1;
      // partner half's raw elements (exchanged by every lane, outside the divergent branch)
      u32x4 xo[NMF];
#pragma unroll
      for (int m = 0; m < NMF; ++m)
#pragma unroll
        for (int w = 0; w < 4; ++w) xo[m][w] = __shfl_xor(xr[tt][m][w], 32, 64);
      if (rerank) {
        // exact fp64 brute force over all codewords (sequential sum, no fused multiply-add)
        double x[E];
#pragma unroll
        for (int m = 0; m < NMF; ++m) {
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const uint32_t h0 = half == 0 ? xr[tt][m][w] : xo[m][w];   // elements 16m + 2w, +1
            const uint32_t h1 = half == 0 ? xo[m][w] : xr[tt][m][w];   // elements 16m + 8 + 2w, +1
            x[16 * m + 2 * w] = (double)bf16_lo(h0);
            x[16 * m + 2 * w + 1] = (double)bf16_hi(h0);
            x[16 * m + 8 + 2 * w] = (double)bf16_lo(h1);
            x[16 * m + 8 + 2 * w + 1] = (double)bf16_hi(h1);
          }
        }
        double bd = INFINITY;
        for (int k = 0; k < kCodes; ++k) {
          const uint16_t* ck = cb_g + k * E;
          double dd = 0.0;
#pragma unroll
          for (int e = 0; e < E; ++e) {
            const double diff = __dsub_rn(x[e], (double)bf16_at(ck + e));
            dd = __dadd_rn(dd, __dmul_rn(diff, diff));
          }
          if (dd < bd) {
            bd = dd;
            best = k;
          }
        }
        if (p.rerank_count && half == 0) atomicAdd(p.rerank_count, 1ull);
      } else if (!rvalid[tt]) {
        continue;
      }
      const int r = row0 + tt * 32 + col;
      if (half == 0 && rvalid[tt]) {
        if (p.out_idx) p.out_idx[((int64_t)r * p.Hkv + h) * NG + g] = best;
        const int seq = p.seq_id[r];
        const int u = p.vq_pos[r];
        if (seq >= 0 && seq < p.batch && u >= 0 && (u >> p.pt_shift) < p.max_pages) {
          const int page = p.block_table[(int64_t)seq * p.max_pages + (u >> p.pt_shift)];
          if (page >= 0 && page < p.num_pages) {
            const int w = u & pt_mask;
            const int64_t off = (int64_t)page * p.page_bytes + (int64_t)p.kind * p.kind_bytes +
                                ((w >> 2) * (NG >> 2) + (g >> 2)) * 16 + (w & 3) * 4 + (g & 3);
            pool_h[off] = (uint8_t)best;
          }
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_encode(const EncodeParams& p, int c, hipStream_t stream) {
  if (p.n_tokens == 0) return hipSuccess;
  const dim3 grid((p.n_tokens + 63) / 64, p.Hkv);
  if (c == 4)
    hipLaunchKernelGGL(encode_kernel<4>, grid, dim3(256), 0, stream, p);
  else if (c == 8)
    hipLaunchKernelGGL(encode_kernel<8>, grid, dim3(256), 0, stream, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace lvq
