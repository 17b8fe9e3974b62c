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
//  * one workgroup = one query x one token split; 4 waves.
//  * prologue: q' = scale*log2(e) * R^T q; then the q.codeword lookup table
//    LUT[k][g] = q'_g . slice_tau(C_k[g]) is built in LDS (K x NG fp32).
//  * LDS row per codeword k (256 B): LUT entries at byte 4*g (NG=32) or two
//    copies at 4*g and 64 + 4*g (NG=16, so 64 lanes cover all 32 banks), and
//    the value histogram at byte 128 + the same offsets.  The LDS address of
//    (k, g) is k*256 + byte(g): one v_perm_b32 places the packed index byte
//    next to the lane's group byte, so an index costs one VALU op + one LDS op.
//  * index stream: a wave reads one 1 KB block of K indices and one of V
//    indices per tile (32 tokens at NG=32, 64 at NG=16), 16 B per lane.  Lane
//    (Q, u) holds 4 tokens x 4 groups; its 16 lookups walk the groups in an
//    order rotated by Q so the lanes of one instruction hit distinct banks.
//  * token scores: per-lane partial sums + a 2-3 step DPP reduce-scatter over
//    the lanes of a token quad, so each lane ends with one full token score.
//  * softmax: scores live in log2 units; p = exp2(s - m_ref) with m_ref the
//    maximum over the first tile of every wave, capped at 2^64.  A split where
//    any later score exceeds m_ref by more than 64 is recomputed with the exact
//    maximum (rare; keeps fp32 sums finite with no per-tile rescaling of the
//    histogram).
//  * values: H[idx_V[n][g]][g] += p_n with LDS float atomics; after the token
//    loop, o[g*c + i] = sum_k H[k][g] * Cv_tau[k][g*c + i] (K*d MACs per split).
//  * bf16 windows: lane-per-token scores, then lane-per-channel value sums.
//  * splits write (m, l, o) partials; a second kernel merges them with
//    log-sum-exp.  One split writes the output directly.
#include "lvq_common.h"

#include <math.h>

namespace lvq {
namespace {

constexpr int kRowBytes = 256;
constexpr int kHOff = 128;
constexpr float kThr = 64.f;
constexpr float kNegInf = -INFINITY;

template <int D, int WAVES>
struct DecodeSmem {
  uint8_t tab[kCodes * kRowBytes];       // LUT + histogram rows (must stay first: LDS offset 0)
  float q[D];                            // q' (log2 units)
  float red[WAVES * 64 > D ? WAVES * 64 : D];  // raw q, then contraction partials
  float wo[WAVES][D];                    // window partial o per wave
  float wm[WAVES], wl[WAVES];            // window partial max / sum per wave
  float vm[WAVES], vl[WAVES];            // VQ max / sum per wave
  int vover[WAVES];
};

__device__ __forceinline__ u32x4 ntload(const u32x4* ptr) { return __builtin_nontemporal_load(ptr); }

__device__ __forceinline__ float lds_f32(const uint8_t* tab, uint32_t addr) {
  return *reinterpret_cast<const float*>(tab + addr);
}

template <int NG, int C, int WAVES>
__global__ void __launch_bounds__(WAVES * 64, 2) decode_kernel(DecodeParams p) {
  constexpr int D = NG * C;
  constexpr int G4 = NG / 4;        // lanes that share a token quad
  constexpr int TW = 256 / G4;      // tokens per wave tile (1 KB of 8-bit indices)
  constexpr int NT = WAVES * 64;
  constexpr int CPL = D / 64;       // window channels per lane
  static_assert(NG == 16 || NG == 32, "NG");
  static_assert(CPL == 1 || CPL == 2 || CPL == 4, "D");

  __shared__ DecodeSmem<D, WAVES> sm;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int Q_total = p.B * p.Hq;
  const int qi = blockIdx.x / p.S;
  const int s = blockIdx.x - qi * p.S;
  const int b = qi / p.Hq;
  const int hq = qi - b * p.Hq;
  const int h = hq / (p.Hq / p.Hkv);

  int N = p.seq_lens[b];
  N = N < 0 ? 0 : (N > p.max_seq_len ? p.max_seq_len : N);
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
  const int t0 = (int)(((int64_t)n_tiles * s) / p.S);
  const int t1 = (int)(((int64_t)n_tiles * (s + 1)) / p.S);
  const bool has_vq = t1 > t0;

  // ---- 1. q' = scale*log2(e) * R^T q -------------------------------------------------
  float* qraw = sm.red;
  if (tid < D) qraw[tid] = bf16_at(p.q + (int64_t)qi * D + tid);
  __syncthreads();
  if (tid < D) {
    float v;
    if (p.rot) {
      v = 0.f;
      for (int i = 0; i < D; ++i) v = fmaf(p.rot[i * D + tid], qraw[i], v);
    } else {
      v = qraw[tid];
    }
    sm.q[tid] = v * p.scale_log2;
  }
  __syncthreads();

  // ---- 2. lookup table and zeroed histogram ---------------------------------------------
  if (has_vq) {
    const uint16_t* sk = p.cbk + ((int64_t)h * p.G + p.tau) * kCodes * D;
    const int g = tid % NG;               // fixed per thread (NT is a multiple of NG)
    float qg[C];
#pragma unroll
    for (int i = 0; i < C; ++i) qg[i] = sm.q[g * C + i];
#pragma unroll 4
    for (int e = tid; e < kCodes * NG; e += NT) {
      const int k = e / NG;
      const uint16_t* src = sk + k * D + g * C;
      float acc = 0.f;
      if constexpr (C == 4) {
        const uint2 w = *reinterpret_cast<const uint2*>(src);
        acc = fmaf(qg[0], bf16_lo(w.x), acc);
        acc = fmaf(qg[1], bf16_hi(w.x), acc);
        acc = fmaf(qg[2], bf16_lo(w.y), acc);
        acc = fmaf(qg[3], bf16_hi(w.y), acc);
      } else {
        const uint4 w = *reinterpret_cast<const uint4*>(src);
        acc = fmaf(qg[0], bf16_lo(w.x), acc);
        acc = fmaf(qg[1], bf16_hi(w.x), acc);
        acc = fmaf(qg[2], bf16_lo(w.y), acc);
        acc = fmaf(qg[3], bf16_hi(w.y), acc);
        acc = fmaf(qg[4], bf16_lo(w.z), acc);
        acc = fmaf(qg[5], bf16_hi(w.z), acc);
        acc = fmaf(qg[6], bf16_lo(w.w), acc);
        acc = fmaf(qg[7], bf16_hi(w.w), acc);
      }
      float* row = reinterpret_cast<float*>(sm.tab + k * kRowBytes);
      row[g] = acc;
      if constexpr (NG == 16) row[16 + g] = acc;
    }
    for (int e = tid; e < kCodes * 32; e += NT)
      reinterpret_cast<float*>(sm.tab + (e >> 5) * kRowBytes + kHOff)[e & 31] = 0.f;
  }

  // ---- 3. bf16 window rows (prefix + recent) of this split ------------------------------
  float m_w = kNegInf, l_w = 0.f, o_w[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) o_w[c] = 0.f;
  {
    const int64_t pre_row0 = ((int64_t)b * p.Hkv + h) * p.P;
    const int64_t rec_row0 = ((int64_t)b * p.Hkv + h) * p.R;
    for (int cbase = w0 + wave * 64; cbase < w1; cbase += NT) {
      const int w = cbase + lane;
      const bool ok = w < w1;
      float sc = kNegInf;
      if (ok) {
        const uint16_t* kr = (w < n_prefix) ? p.k_prefix + (pre_row0 + w) * D
                                            : p.k_recent + (rec_row0 + (w - n_prefix)) * D;
        float acc = 0.f;
#pragma unroll
        for (int c8 = 0; c8 < D / 8; ++c8) {
          const uint4 kv = *reinterpret_cast<const uint4*>(kr + c8 * 8);
          const float* qq = sm.q + c8 * 8;
          acc = fmaf(qq[0], bf16_lo(kv.x), acc);
          acc = fmaf(qq[1], bf16_hi(kv.x), acc);
          acc = fmaf(qq[2], bf16_lo(kv.y), acc);
          acc = fmaf(qq[3], bf16_hi(kv.y), acc);
          acc = fmaf(qq[4], bf16_lo(kv.z), acc);
          acc = fmaf(qq[5], bf16_hi(kv.z), acc);
          acc = fmaf(qq[6], bf16_lo(kv.w), acc);
          acc = fmaf(qq[7], bf16_hi(kv.w), acc);
        }
        sc = acc;
      }
      const float mc = wave_max(sc);
      const float mn = fmaxf(m_w, mc);
      const float a = __builtin_amdgcn_exp2f(m_w - mn);
      const float pn = ok ? __builtin_amdgcn_exp2f(sc - mn) : 0.f;
      l_w = l_w * a + wave_sum(pn);
#pragma unroll
      for (int c = 0; c < CPL; ++c) o_w[c] *= a;
      m_w = mn;
      const int cnt = (w1 - cbase) < 64 ? (w1 - cbase) : 64;
#pragma unroll 8
      for (int n = 0; n < cnt; ++n) {
        const float pv = __shfl(pn, n, 64);
        const int wn = cbase + n;
        const uint16_t* vr = (wn < n_prefix) ? p.v_prefix + (pre_row0 + wn) * D
                                             : p.v_recent + (rec_row0 + (wn - n_prefix)) * D;
        if constexpr (CPL == 1) {
          o_w[0] = fmaf(pv, bf16_at(vr + lane), o_w[0]);
        } else if constexpr (CPL == 2) {
          const uint32_t v2 = *reinterpret_cast<const uint32_t*>(vr + 2 * lane);
          o_w[0] = fmaf(pv, bf16_lo(v2), o_w[0]);
          o_w[1] = fmaf(pv, bf16_hi(v2), o_w[1]);
        } else {
          const uint2 v4 = *reinterpret_cast<const uint2*>(vr + 4 * lane);
          o_w[0] = fmaf(pv, bf16_lo(v4.x), o_w[0]);
          o_w[1] = fmaf(pv, bf16_hi(v4.x), o_w[1]);
          o_w[2] = fmaf(pv, bf16_lo(v4.y), o_w[2]);
          o_w[3] = fmaf(pv, bf16_hi(v4.y), o_w[3]);
        }
      }
    }
  }
  if (lane == 0) {
    sm.wm[wave] = m_w;
    sm.wl[wave] = l_w;
  }
#pragma unroll
  for (int c = 0; c < CPL; ++c) sm.wo[wave][lane * CPL + c] = o_w[c];

  __syncthreads();   // LUT, histogram zeroing and window partials complete

  // ---- 4. vector-quantized rows ---------------------------------------------------------
  float m_ref = kNegInf, l_vq = 0.f;
  if (has_vq) {
    const int Qd = lane / G4, u = lane % G4;
    uint32_t base[4], sel[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t gg = 4u * u + ((r + Qd) & 3);
      base[r] = gg * 4u + ((NG == 16) ? (uint32_t)(Qd & 1) * 64u : 0u);
      sel[r] = 0x0c0c0000u | ((4u + ((r + Qd) & 3)) << 8);
    }
    const int tok = (NG == 16) ? u : (((u >= 4) ? 2 : 0) + ((u & 2) ? 1 : 0));
    const bool hi = (u >= 4);
    const uint8_t* pool_h = p.pool_lj + (int64_t)h * p.head_stride;
    const int32_t* bt = p.block_table + (int64_t)b * p.max_pages;
    const int pt_mask = (1 << p.pt_shift) - 1;

    auto tile_ptr = [&](int t) -> const uint8_t* {
      const int u0 = t * TW;
      int pg = bt[u0 >> p.pt_shift];
      if (pg < 0 || pg >= p.num_pages) pg = 0;
      return pool_h + (int64_t)pg * p.page_bytes + (int64_t)(u0 & pt_mask) * NG + lane * 16;
    };

    auto score = [&](const u32x4 xk, int t) -> float {
      const uint32_t xs[4] = {xk.x, xk.y, xk.z, xk.w};
      float acc[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float a = lds_f32(sm.tab, __builtin_amdgcn_perm(xs[i], base[0], sel[0]));
#pragma unroll
        for (int r = 1; r < 4; ++r) a += lds_f32(sm.tab, __builtin_amdgcn_perm(xs[i], base[r], sel[r]));
        acc[i] = a;
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
        const float k0 = hi ? acc[2] : acc[0], s0 = hi ? acc[0] : acc[2];
        const float k1 = hi ? acc[3] : acc[1], s1 = hi ? acc[1] : acc[3];
        const float c0 = k0 + dpp<kDppRowHalfMirror>(s0);
        const float c1 = k1 + dpp<kDppRowHalfMirror>(s1);
        const bool b2 = (u & 2) != 0;
        const float kk = b2 ? c1 : c0, ss = b2 ? c0 : c1;
        const float d0 = kk + dpp<dpp_quad(2, 3, 0, 1)>(ss);
        sc = d0 + dpp<dpp_quad(1, 0, 3, 2)>(d0);
      }
      const bool valid = t * TW + 4 * Qd + tok < n_vq;
      return valid ? sc : kNegInf;
    };

    auto accum_v = [&](const u32x4 xv, float pp) {
      float pi[4];
      if constexpr (NG == 16) {
        pi[0] = dpp<dpp_quad(0, 0, 0, 0)>(pp);
        pi[1] = dpp<dpp_quad(1, 1, 1, 1)>(pp);
        pi[2] = dpp<dpp_quad(2, 2, 2, 2)>(pp);
        pi[3] = dpp<dpp_quad(3, 3, 3, 3)>(pp);
      } else {
        const float a = dpp<dpp_quad(0, 0, 0, 0)>(pp);
        const float bb = dpp<dpp_quad(2, 2, 2, 2)>(pp);
        const float am = dpp<kDppRowHalfMirror>(a);
        const float bm = dpp<kDppRowHalfMirror>(bb);
        pi[0] = hi ? am : a;
        pi[1] = hi ? bm : bb;
        pi[2] = hi ? a : am;
        pi[3] = hi ? bb : bm;
      }
      const uint32_t xs[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const uint32_t addr = __builtin_amdgcn_perm(xs[i], base[r], sel[r]);
          atomicAdd(reinterpret_cast<float*>(sm.tab + addr + kHOff), pi[i]);
        }
      }
    };

    const int my_first = t0 + wave;
    const int n_my = (my_first < t1) ? (t1 - my_first + WAVES - 1) / WAVES : 0;

    // reference maximum: the first tile of every wave
    float m_loc = kNegInf;
    if (n_my > 0) {
      const u32x4 xk = ntload(reinterpret_cast<const u32x4*>(tile_ptr(my_first)));
      m_loc = wave_max(score(xk, my_first));
    }
    if (lane == 0) sm.vm[wave] = m_loc;
    __syncthreads();
    m_ref = sm.vm[0];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) m_ref = fmaxf(m_ref, sm.vm[w]);
    __syncthreads();

    for (int pass = 0; pass < 2; ++pass) {
      float lsum = 0.f, smax = kNegInf;
      bool over = false;
      auto process = [&](const u32x4 xk, const u32x4 xv, int t) {
        const float sc = score(xk, t);
        smax = fmaxf(smax, sc);
        const float e = sc - m_ref;
        over |= e > kThr;
        const float pp = __builtin_amdgcn_exp2f(fminf(e, kThr));
        lsum += (NG == 32 && (u & 1)) ? 0.f : pp;
        accum_v(xv, pp);
      };
      // rotating prefetch of kPF tiles per wave (K and V index blocks)
      constexpr int kPF = 4;
      u32x4 bk[kPF], bv[kPF];
      if (n_my > 0) {
#pragma unroll
      for (int j = 0; j < kPF; ++j) {
        const uint8_t* pa = tile_ptr(my_first + (j < n_my ? j : n_my - 1) * WAVES);
        bk[j] = ntload(reinterpret_cast<const u32x4*>(pa));
        bv[j] = ntload(reinterpret_cast<const u32x4*>(pa + p.kind_bytes));
      }
      // steady state: branch-free, every slot is refilled (clamped to the last tile, so the
      // refills past the end re-read a valid tile and are never consumed)
      const int n_full = n_my - n_my % kPF;
      for (int i0 = 0; i0 < n_full; i0 += kPF) {
#pragma unroll
        for (int j = 0; j < kPF; ++j) {
          // keep each slot's work in program order: hoisting a later slot's index
          // arithmetic above this point would stall on that slot's in-flight load
          __builtin_amdgcn_sched_barrier(0);
          process(bk[j], bv[j], my_first + (i0 + j) * WAVES);
          const int inext = (i0 + j + kPF < n_my) ? (i0 + j + kPF) : (n_my - 1);
          const uint8_t* pa = tile_ptr(my_first + inext * WAVES);
          bk[j] = ntload(reinterpret_cast<const u32x4*>(pa));
          bv[j] = ntload(reinterpret_cast<const u32x4*>(pa + p.kind_bytes));
        }
      }
#pragma unroll
      for (int j = 0; j < kPF - 1; ++j)
        if (n_full + j < n_my) process(bk[j], bv[j], my_first + (n_full + j) * WAVES);
      }
      lsum = wave_sum(lsum);
      smax = wave_max(smax);
      const bool wover = __any(over);
      if (lane == 0) {
        sm.vl[wave] = lsum;
        sm.vm[wave] = smax;
        sm.vover[wave] = wover ? 1 : 0;
      }
      __syncthreads();
      int any_over = 0;
      float all_max = kNegInf;
      l_vq = 0.f;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) {
        any_over |= sm.vover[w];
        all_max = fmaxf(all_max, sm.vm[w]);
        l_vq += sm.vl[w];
      }
      if (!any_over || pass == 1) break;
      // rare: a score exceeded the reference by more than 2^64; redo with the exact maximum
      m_ref = all_max;
      __syncthreads();
      for (int e = tid; e < kCodes * 32; e += NT)
        reinterpret_cast<float*>(sm.tab + (e >> 5) * kRowBytes + kHOff)[e & 31] = 0.f;
      __syncthreads();
    }
  }

  // ---- 5. value contraction o_vq = H^T Cv_tau, merge, write -----------------------------
  constexpr int PARTS = NT / D;
  float o_vq = 0.f;
  if (has_vq) {
    const int ch = tid % D, part = tid / D, g = ch / C;
    const uint16_t* sv = p.cbv + ((int64_t)h * p.G + p.tau) * kCodes * D + ch;
    float acc = 0.f;
#pragma unroll 16
    for (int k = part; k < kCodes; k += PARTS) {
      const float* row = reinterpret_cast<const float*>(sm.tab + k * kRowBytes + kHOff);
      float hk = row[g];
      if constexpr (NG == 16) hk += row[16 + g];
      acc = fmaf(hk, bf16_at(sv + k * D), acc);
    }
    sm.red[tid] = acc;
  }
  __syncthreads();
  if (tid < D) {
    if (has_vq) {
#pragma unroll
      for (int pp = 0; pp < PARTS; ++pp) o_vq += sm.red[pp * D + tid];
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
      p.out[(int64_t)qi * D + tid] = ot / lt;
      if (p.lse && tid == 0) p.lse[qi] = M * 0.6931471805599453f + logf(lt);
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
  p.out[(int64_t)qi * D + tid] = ot / lt;
  if (p.lse && tid == 0) p.lse[qi] = M * 0.6931471805599453f + logf(lt);
}

template <int NG, int C>
hipError_t launch_variant(const DecodeParams& p, hipStream_t stream) {
  constexpr int WAVES = 4;
  const int Q = p.B * p.Hq;
  hipLaunchKernelGGL((decode_kernel<NG, C, WAVES>), dim3(Q * p.S), dim3(WAVES * 64), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.S == 1) return e;
  hipLaunchKernelGGL((combine_kernel<NG * C>), dim3(Q), dim3(NG * C), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, int ng, int c, hipStream_t stream) {
  if (ng == 32 && c == 4) return launch_variant<32, 4>(p, stream);
  if (ng == 16 && c == 4) return launch_variant<16, 4>(p, stream);
  if (ng == 16 && c == 8) return launch_variant<16, 8>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace lvq
