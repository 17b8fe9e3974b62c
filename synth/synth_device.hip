// Device twin of synth/gen.py: regenerates the same bf16 K/V cache values on the GPU,
// bit for bit, for workloads too large to build on the host.
//
// Input generation only (no LoopVQ arithmetic).  The steps and their order follow
// gen.py exactly: SplitMix64 at a position -> 16-bit field -> normal quantile table
// -> AR(1) along loop steps in fp64 (two rounded products, one rounded sum) ->
// per-channel scale -> optional key rotation (sign flip, fast Walsh-Hadamard
// transform with stages 1, 2, 4, ..., one rounded product by 1/sqrt(d)) -> fp32 ->
// bf16, both roundings to nearest even.  Every fp64 operation is written with an
// explicit rounding intrinsic so no multiply-add is contracted.
#include <hip/hip_runtime.h>
#include <stdint.h>

extern "C" {
typedef struct synth_kv_args {
  uint64_t key;                 /* stream key of the data stream */
  const double* table;          /* device fp64[65536] normal quantiles */
  const double* scales;         /* device fp64 [L][Hkv][2][d] */
  const double* signs;          /* device fp64 [d] rotation signs, or NULL (no rotation) */
  double inv_sqrt_d, rho, innov;
  int32_t T4;                   /* loop count rounded up to a multiple of 4 */
  int32_t L, B, Hkv, n_ctx, d;  /* counter layout */
  int32_t kind, layer;
  int32_t b0, nb, h0, nh;       /* sequences [b0, b0+nb), kv-heads [h0, h0+nh) */
  int32_t n0, nn;               /* tokens [n0, n0+nn) */
  int32_t t0, nt;               /* loop steps [t0, t0+nt) written */
  uint16_t* out;                /* device bf16 */
  int64_t s_loop, s_b, s_h, s_n;/* element strides of out (channel stride 1) */
} synth_kv_args;
int synth_kv(const synth_kv_args* a, void* stream);
}

namespace {

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ __forceinline__ double normal_at(uint64_t key, uint64_t j, const double* table) {
  const uint64_t u = mix64(key + ((j >> 2) + 1ull) * 0x9E3779B97F4A7C15ull);
  return table[(u >> ((j & 3ull) * 16ull)) & 0xFFFFull];
}

__device__ __forceinline__ uint16_t to_bf16(double x) {
  const uint32_t u = __float_as_uint((float)x);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// one block per (b, h, n) row, one thread per channel
__global__ void synth_kv_kernel(synth_kv_args a) {
  extern __shared__ double buf[];   // 2 * d
  const int ch = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int n = a.n0 + (int)(row % a.nn);
  const int64_t r2 = row / a.nn;
  const int h = a.h0 + (int)(r2 % a.nh);
  const int b = a.b0 + (int)(r2 / a.nh);
  const uint64_t e = ((((uint64_t)(a.kind * a.L + a.layer) * a.B + b) * a.Hkv + h) * a.n_ctx + n) * a.d + ch;
  const double s = a.scales[(((int64_t)a.layer * a.Hkv + h) * 2 + a.kind) * a.d + ch];
  const bool rot = a.signs != nullptr && a.kind == 0;
  double x = 0.0;
  for (int t = 0; t < a.t0 + a.nt; ++t) {
    const double eps = normal_at(a.key, e * (uint64_t)a.T4 + (uint64_t)t, a.table);
    x = (t == 0) ? eps : __dadd_rn(__dmul_rn(a.rho, x), __dmul_rn(a.innov, eps));
    if (t < a.t0) continue;
    double v = __dmul_rn(s, x);
    if (rot) {
      double* cur = buf;
      double* nxt = buf + a.d;
      cur[ch] = __dmul_rn(v, a.signs[ch]);
      __syncthreads();
      for (int hh = 1; hh < a.d; hh <<= 1) {
        const double va = cur[ch & ~hh], vb = cur[ch | hh];
        nxt[ch] = (ch & hh) ? __dsub_rn(va, vb) : __dadd_rn(va, vb);
        __syncthreads();
        double* tmp = cur;
        cur = nxt;
        nxt = tmp;
      }
      v = __dmul_rn(cur[ch], a.inv_sqrt_d);
      __syncthreads();
    }
    a.out[(int64_t)(t - a.t0) * a.s_loop + (int64_t)(b - a.b0) * a.s_b + (int64_t)(h - a.h0) * a.s_h +
          (int64_t)(n - a.n0) * a.s_n + ch] = to_bf16(v);
  }
}

}  // namespace

extern "C" int synth_kv(const synth_kv_args* a, void* stream) {
  if (!a || !a->table || !a->scales || !a->out || a->d < 1 || a->d > 1024 || (a->d & (a->d - 1)) || a->nb < 0 ||
      a->nh < 0 || a->nn < 0 || a->nt < 0 || a->t0 < 0 || a->t0 + a->nt > a->T4)
    return -1;
  const int64_t rows = (int64_t)a->nb * a->nh * a->nn;
  if (rows == 0 || a->nt == 0) return 0;
  if (rows > 0x7fffffffLL) return -1;
  hipLaunchKernelGGL(synth_kv_kernel, dim3((unsigned)rows), dim3(a->d), 2 * a->d * sizeof(double),
                     (hipStream_t)stream, *a);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}
