// Codebook preparation: the decode-side copy and the encode-side squared norms.
//
// Canonical codebooks are [set][g][k][tau*c + i] (one row per codeword, loop-major
// sub-vector order).  Decode at loop step t reads only the (t mod G) slice of every
// codeword, so the prepared copy is [set][tau][k][g*c + i]: the slice of one set is a
// contiguous K x d block, read with the same stride as a cache row.  The squared
// norms ||C_k||^2 (fp32, summed in element order) seed the encode screen.
#include "lvq_common.h"

namespace lvq {
namespace {

__global__ void __launch_bounds__(256) prepare_slices(PrepareParams p) {
  const int64_t total = p.sets * p.G * p.K * p.d;
  const int E = p.c * p.G;
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total; idx += (int64_t)gridDim.x * 256) {
    const int ch = (int)(idx % p.d);
    const int64_t r1 = idx / p.d;
    const int k = (int)(r1 % p.K);
    const int64_t r2 = r1 / p.K;
    const int tau = (int)(r2 % p.G);
    const int64_t set = r2 / p.G;
    const int g = ch / p.c, i = ch - g * p.c;
    p.prep[idx] = p.cb[((set * p.NG + g) * p.K + k) * E + tau * p.c + i];
  }
}

// Group-major loop slices for extend: [set][tau][g][k][i].  A gather of one group's channels of
// codeword k then stays inside that group's K x c block (2 KB at c=4), so the gathers of a tile
// touch few cache lines.
__global__ void __launch_bounds__(256) prepare_groups(PrepareParams p) {
  const int64_t total = p.sets * p.G * p.NG * p.K * p.c;
  const int E = p.c * p.G;
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total; idx += (int64_t)gridDim.x * 256) {
    const int i = (int)(idx % p.c);
    const int64_t r1 = idx / p.c;
    const int k = (int)(r1 % p.K);
    const int64_t r2 = r1 / p.K;
    const int g = (int)(r2 % p.NG);
    const int64_t r3 = r2 / p.NG;
    const int tau = (int)(r3 % p.G);
    const int64_t set = r3 / p.G;
    p.prep[idx] = p.cb[((set * p.NG + g) * p.K + k) * E + tau * p.c + i];
  }
}

__global__ void __launch_bounds__(256) prepare_norms(PrepareParams p) {
  const int64_t total = p.sets * p.NG * p.K;
  const int E = p.c * p.G;
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total; idx += (int64_t)gridDim.x * 256) {
    p.norms[idx] = codeword_norm(p.cb + idx * E, E);
  }
}

}  // namespace

hipError_t launch_prepare_groups(const PrepareParams& p, hipStream_t stream) {
  const int64_t n = p.sets * p.G * p.NG * p.K * p.c;
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(prepare_groups, dim3((unsigned)(blocks < 65536 ? blocks : 65536)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_prepare(const PrepareParams& p, hipStream_t stream) {
  const int64_t n1 = p.sets * p.G * p.K * p.d;
  const int64_t b1 = (n1 + 255) / 256;
  hipLaunchKernelGGL(prepare_slices, dim3((unsigned)(b1 < 65536 ? b1 : 65536)), dim3(256), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !p.norms) return e;
  const int64_t n2 = p.sets * p.NG * p.K;
  const int64_t b2 = (n2 + 255) / 256;
  hipLaunchKernelGGL(prepare_norms, dim3((unsigned)(b2 < 65536 ? b2 : 65536)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace lvq
