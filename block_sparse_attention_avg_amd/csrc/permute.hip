// Token reorder (NABLA summary, Metodologia section 1, fractal flattening;
// Sparse VideoGen2 summary, Metodologia A, semantic permutation and its
// inverse). Pure data movement: every thread moves one 16-byte chunk of a
// token row, consecutive threads walk consecutive chunks of a row so both the
// gather and the scatter side are full 128-byte lines. HBM-bound:
// 2 * N * d * 2 bytes per (b, h).
#include "common.h"

namespace bsa {

template <int CPR>
__global__ __launch_bounds__(256) void permute_kernel(const uint4* __restrict__ x,
                                                     uint4* __restrict__ y,
                                                     const int32_t* __restrict__ perm, int N,
                                                     int per_head, int inverse) {
  const int bh = blockIdx.y;
  const size_t u = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (u >= (size_t)N * CPR) return;
  const int i = (int)(u / CPR), c = (int)(u % CPR);
  const int p = perm[(per_head ? (size_t)bh * N : 0) + i];
  const size_t base = (size_t)bh * N;
  if (!inverse)
    y[(base + i) * CPR + c] = x[(base + p) * CPR + c];
  else
    y[(base + p) * CPR + c] = x[(base + i) * CPR + c];
}

hipError_t launch_permute(const uint16_t* x, uint16_t* y, const int32_t* perm, int BH, int N,
                          int d, int per_head, bool inverse, hipStream_t s) {
  if (BH == 0 || N == 0) return hipSuccess;
  const int cpr = d / 8;
  dim3 grid((unsigned)(((size_t)N * cpr + 255) / 256), BH);
  const uint4* xs = reinterpret_cast<const uint4*>(x);
  uint4* ys = reinterpret_cast<uint4*>(y);
  switch (cpr) {
    case 16: permute_kernel<16><<<grid, 256, 0, s>>>(xs, ys, perm, N, per_head, inverse); break;
    case 8: permute_kernel<8><<<grid, 256, 0, s>>>(xs, ys, perm, N, per_head, inverse); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace bsa
