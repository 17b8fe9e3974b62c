// One weighted Lloyd iteration for one codebook set (airadar.tv LoopVQ summary, opening
// summary: the codebooks come from k-means weighted by Fisher information).  The
// assignment is the encode kernel run without a pool; two kernels here turn it into the
// new codebook:
//
//   lloyd_sums    per (row chunk, kv-head, loop step tau, 64-channel slice): for every
//                 codeword, the sum of w * x over its samples, per element, accumulated in
//                 LDS in fp64 (the product of an fp32 weight and a bf16 element is exact in
//                 fp64); the total weight W_k of the codewords of the slice's groups with
//                 g = tau (mod G), so that the G loop-step workgroups of a slice share that
//                 work; and the sum of w * ||x||^2 per group.  One partial per workgroup,
//                 written with plain stores.
//   lloyd_update  per codeword: adds the partials in a fixed order, divides, rounds the mean
//                 to bf16 (nearest, ties to even, straight from fp64) and recomputes the
//                 codeword's squared norm; a codeword with no weight keeps its value.  The
//                 weighted distortion of the old codebook follows without a second pass:
//                 sum_k sum_{r in k} w ||x_r - C_k||^2
//                   = sum_r w ||x_r||^2 - sum_k (2 C_k . S_k - W_k ||C_k||^2),  S_k = sum w x
//
// A workgroup of lloyd_sums reads 128 contiguous bytes (64 channels of one loop-step plane)
// of each of its rows, so every HBM line it touches is used whole.  Its LDS accumulator is
// [codeword][channel] fp64 (128 KB), and the lanes of each atomic add are given channels
// that fall on distinct banks whatever the codewords.
#include "lvq_common.h"

namespace lvq {
namespace {

constexpr int kCodesL = 256;
constexpr int kSliceCh = 64;

// fp64 -> bf16, round to nearest even, without double rounding: the fp32 intermediate is
// rounded to odd (truncate, then set the last bit if anything was dropped), which keeps
// enough information for the second rounding to be the correct one (Boldo and Melquiond,
// "Emulation of FMA and correctly rounded sums: proved algorithms using rounding to odd").
__device__ __forceinline__ uint16_t bf16_from_f64(double v) {
  const float f = __double2float_rz(v);
  uint32_t u = __float_as_uint(f);
  if ((double)f != v) u |= 1u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <int C, bool DIST>
__global__ void __launch_bounds__(1024, 1) lloyd_sums(LloydParams p) {
  constexpr int GPS = kSliceCh / C;          // groups in a slice
  constexpr int GPL = 8 / C;                 // groups per lane (8 channels per lane)
  constexpr int ACC = GPS * C * kCodesL;     // 16384 doubles
  constexpr int WG_MAX = GPS / 2;            // weight groups per workgroup (G >= 2)
  constexpr int U = 4;                       // rows per lane in flight
  __shared__ __align__(16) double acc[ACC];
  __shared__ double wacc[WG_MAX * kCodesL];
  __shared__ double dacc[GPS];
  const int slices = p.d / kSliceCh;
  // logical block = (chunk, kv-head, loop step, slice), slice fastest: the workgroups that
  // read one kv-head's assignment and weight rows share an XCD
  const int q = xcd_local_block(blockIdx.x, gridDim.x);
  const int slice = q % slices;
  const int tau = (q / slices) % p.G;
  const int h = (q / (slices * p.G)) % p.Hkv;
  const int chunk = q / (slices * p.G * p.Hkv);
  const int wgroups = GPS / p.G;             // slice groups m * G + tau, m < wgroups
  for (int i = threadIdx.x; i < ACC; i += 1024) acc[i] = 0.0;
  for (int i = threadIdx.x; i < WG_MAX * kCodesL; i += 1024) wacc[i] = 0.0;
  if (threadIdx.x < GPS) dacc[threadIdx.x] = 0.0;
  __syncthreads();

  const int sub = threadIdx.x & 7;           // 8-channel piece of the slice
  const int rs = (threadIdx.x >> 3) & 7;     // row of the lane within its wave's 8 rows
  // Step j of the lane's 8 atomic adds takes its channel e = (j + rot) mod 8.  A 64-bit LDS
  // access is served 16 lanes (32 banks) at a time: lanes 16m..16m+15 are rows {2m, 2m+1} x the
  // 8 pieces, and rot = 4*sub[2] + 2*(sub[1] ^ rs[1]) + rs[0] gives those 16 lanes 16 distinct
  // (channel mod 16), hence distinct banks, whatever the codewords (and 32 distinct channels mod
  // 32 over lanes 32m..32m+31).
  const int rot = (((sub >> 2) & 1) << 2) | ((((sub >> 1) ^ (rs >> 1)) & 1) << 1) | (rs & 1);
  const uint32_t m1 = (rot & 2) ? ~0u : 0u, m2 = (rot & 4) ? ~0u : 0u, sh = (rot & 1) * 16u;
  const int gl0 = sub * GPL;                 // first group of this lane within the slice
  const int g0 = slice * GPS + gl0;
  const int64_t r_begin = (int64_t)chunk * p.rows_a;
  const int64_t r_end = min((int64_t)p.n, r_begin + p.rows_a);
  const uint16_t* xb = p.src + tau * p.stride_loop + h * p.stride_head + slice * kSliceCh + sub * 8;
  bool wown[GPL];                            // this lane adds the weight of its group gl
#pragma unroll
  for (int gl = 0; gl < GPL; ++gl) wown[gl] = (gl0 + gl) % p.G == tau;
  double dpart[GPL];
#pragma unroll
  for (int gl = 0; gl < GPL; ++gl) dpart[gl] = 0.0;

  // rows of one batch: U rows per lane, 128 rows apart; the next batch is loaded while this one's
  // atomic adds run
  struct Batch {
    uint4 xv[U];
    int kk[U][GPL];
    float ww[U][GPL];
  };
  auto load_batch = [&](int64_t rb, int64_t rvalid, Batch& bt) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t r = rb + u * 128;
      const int64_t rr = r < r_end ? r : rvalid;   // rows past the end reload a valid row with weight 0
      bt.xv[u] = *(const uint4*)(xb + rr * p.stride_token);
      const int64_t o = (rr * p.Hkv + h) * p.NG + g0;
      if constexpr (GPL == 2) {
        const int2 k2 = *(const int2*)(p.assign + o);
        const float2 w2 = *(const float2*)(p.weight + o);
        bt.kk[u][0] = k2.x & (kCodesL - 1);
        bt.kk[u][1] = k2.y & (kCodesL - 1);
        bt.ww[u][0] = r < r_end ? w2.x : 0.f;
        bt.ww[u][1] = r < r_end ? w2.y : 0.f;
      } else {
        bt.kk[u][0] = p.assign[o] & (kCodesL - 1);
        bt.ww[u][0] = r < r_end ? p.weight[o] : 0.f;
      }
    }
  };
  const int64_t rb0 = r_begin + (threadIdx.x >> 3);
  Batch cur;
  if (rb0 < r_end) load_batch(rb0, rb0, cur);
  for (int64_t rb = rb0; rb < r_end; rb += 128 * U) {
    Batch nxt;
    load_batch(rb + 128 * U, rb, nxt);
    const uint4* xv = cur.xv;
    int (&kk)[U][GPL] = cur.kk;
    float (&ww)[U][GPL] = cur.ww;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t xw[4] = {xv[u].x, xv[u].y, xv[u].z, xv[u].w};
#pragma unroll
      for (int gl = 0; gl < GPL; ++gl)
        if (wown[gl]) atomicAdd(&wacc[((gl0 + gl) / p.G) * kCodesL + kk[u][gl]], (double)ww[u][gl]);
      if constexpr (DIST) {
#pragma unroll
        for (int gl = 0; gl < GPL; ++gl) {
          double x2 = 0.0;
#pragma unroll
          for (int i = 0; i < C; ++i) {
            const int j = gl * C + i;
            const float xf = (j & 1) ? bf16_hi(xw[j >> 1]) : bf16_lo(xw[j >> 1]);
            x2 += (double)(xf * xf);   // a bf16 square is exact in fp32
          }
          dpart[gl] += (double)ww[u][gl] * x2;
        }
      }
      // The lane's 8 channels are rotated by rot once (element j of the rotated words is channel
      // (j + rot) mod 8), so the adds index registers statically: words rotated by rot >> 1 (bit 1:
      // one word, bit 2: two words), then by half a word when rot is odd.  The selections are bit
      // blends (a select between array elements would become a dynamically indexed array).
      uint32_t t[4], rw[4], xr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) t[i] = xw[i] ^ ((xw[i] ^ xw[(i + 1) & 3]) & m1);
#pragma unroll
      for (int i = 0; i < 4; ++i) rw[i] = t[i] ^ ((t[i] ^ t[(i + 2) & 3]) & m2);
#pragma unroll
      for (int i = 0; i < 4; ++i) xr[i] = __builtin_amdgcn_alignbit(rw[(i + 1) & 3], rw[i], sh);
      int k0 = kk[u][0], kx = 0;
      uint32_t w0 = __float_as_uint(ww[u][0]), wx = 0u;
      if constexpr (GPL == 2) {
        kx = k0 ^ kk[u][1];
        wx = w0 ^ __float_as_uint(ww[u][1]);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int e = (j + rot) & 7;
        const float xf = (j & 1) ? bf16_hi(xr[j >> 1]) : bf16_lo(xr[j >> 1]);
        const int hm = -((e >> 2) & 1);              // all ones for the lane's second group (c = 4)
        const int k = k0 ^ (kx & hm);
        const float w = __uint_as_float(w0 ^ (wx & (uint32_t)hm));
        atomicAdd(&acc[k * kSliceCh + sub * 8 + e], (double)w * (double)xf);
      }
    }
    cur = nxt;
  }
  if constexpr (DIST) {
#pragma unroll
    for (int gl = 0; gl < GPL; ++gl) atomicAdd(&dacc[gl0 + gl], dpart[gl]);
  }
  __syncthreads();
  const int64_t part = ((int64_t)(chunk * p.Hkv + h) * p.G + tau) * slices + slice;
  double2* out = (double2*)(p.part_sums + part * ACC);
  for (int i = threadIdx.x; i < ACC / 2; i += 1024) out[i] = ((const double2*)acc)[i];
  // W_k of the slice groups m * G + tau
  double* wout = p.part_w + ((int64_t)(chunk * p.Hkv + h) * p.NG + slice * GPS + tau) * kCodesL;
  for (int i = threadIdx.x; i < wgroups * kCodesL; i += 1024)
    wout[(int64_t)(i / kCodesL) * p.G * kCodesL + (i % kCodesL)] = wacc[i];
  if (DIST && threadIdx.x < GPS)
    p.part_dist[((int64_t)(chunk * p.Hkv + h) * p.G + tau) * p.NG + slice * GPS + threadIdx.x] = dacc[threadIdx.x];
}

// One workgroup per (kv-head, group), one thread per codeword.
template <int C>
__global__ void __launch_bounds__(256) lloyd_update(LloydParams p) {
  constexpr int GPS = kSliceCh / C;
  __shared__ double red[256];
  const int k = threadIdx.x;
  const int g = blockIdx.x % p.NG, h = blockIdx.x / p.NG;
  const int64_t t = (int64_t)blockIdx.x * kCodesL + k;
  const int slices = p.d / kSliceCh, slice = g / GPS, gl = g % GPS;
  double W = 0.0;
  for (int ch = 0; ch < p.chunks_a; ++ch) W += p.part_w[((int64_t)(ch * p.Hkv + h) * p.NG + g) * kCodesL + k];
  uint16_t* row = p.cb + t * p.E;
  double cs = 0.0, cc = 0.0;   // C_k . S_k and ||C_k||^2 of the old codeword
  if (W > 0.0) {
    for (int tau = 0; tau < p.G; ++tau) {
      double S[C];
#pragma unroll
      for (int i = 0; i < C; ++i) S[i] = 0.0;
      for (int ch = 0; ch < p.chunks_a; ++ch) {
        const int64_t part = ((int64_t)(ch * p.Hkv + h) * p.G + tau) * slices + slice;
        const double* s = p.part_sums + part * (GPS * C * kCodesL) + k * kSliceCh + gl * C;
#pragma unroll
        for (int i = 0; i < C; ++i) S[i] += s[i];
      }
#pragma unroll
      for (int i = 0; i < C; ++i) {
        const double old = (double)bf16_at(row + tau * C + i);
        cs += old * S[i];
        cc += old * old;
        row[tau * C + i] = bf16_from_f64(S[i] / W);
      }
    }
  }
  p.norms[t] = codeword_norm(row, p.E);
  if (p.cluster_weight) p.cluster_weight[t] = W;
  if (p.distortion) {
    red[k] = W * cc - 2.0 * cs;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
      if (k < s) red[k] += red[k + s];
      __syncthreads();
    }
    if (k == 0) {
      double D = red[0];
      for (int ch = 0; ch < p.chunks_a; ++ch)
        for (int tau = 0; tau < p.G; ++tau) D += p.part_dist[((int64_t)(ch * p.Hkv + h) * p.G + tau) * p.NG + g];
      p.distortion[(int64_t)h * p.NG + g] = D;
    }
  }
}

}  // namespace

hipError_t launch_lloyd(const LloydParams& p, int c, hipStream_t stream) {
  const int slices = p.d / kSliceCh;
  const dim3 ga((unsigned)(p.chunks_a * p.Hkv * p.G * slices));
  const bool dist = p.distortion != nullptr;
  if (c == 4) {
    if (dist) hipLaunchKernelGGL((lloyd_sums<4, true>), ga, dim3(1024), 0, stream, p);
    else hipLaunchKernelGGL((lloyd_sums<4, false>), ga, dim3(1024), 0, stream, p);
  } else {
    if (dist) hipLaunchKernelGGL((lloyd_sums<8, true>), ga, dim3(1024), 0, stream, p);
    else hipLaunchKernelGGL((lloyd_sums<8, false>), ga, dim3(1024), 0, stream, p);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 gu((unsigned)(p.Hkv * p.NG));
  if (c == 4) hipLaunchKernelGGL((lloyd_update<4>), gu, dim3(256), 0, stream, p);
  else hipLaunchKernelGGL((lloyd_update<8>), gu, dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace lvq
