// Block mean pooling of Q or K (NABLA summary, Metodologia section 2,
// "Sottocampionamento": Q and K are average-pooled over N-token blocks).
//
// HBM-bound streaming kernel: one workgroup of 256 threads per block. A row of
// d bf16 values is read as d/8 16-byte chunks; thread t owns chunk t % (d/8)
// and every (256/(d/8))-th row, so each wave reads whole 128-byte lines and a
// 64-token block is fully in flight after one round of loads. Per-thread fp32
// partial sums are combined in LDS in a fixed tree order, so results are
// bit-reproducible. Algorithmic traffic: len*d*2 bytes read + d*4 written per
// block.
#include "common.h"

namespace bsa {

// One tensor per grid z-slice: z = 0 pools (x0, blk0) into out0, z = 1 (when
// given) pools (x1, blk1) into out1, so Q and K take one launch.
template <int D>
__global__ __launch_bounds__(256) void pool_kernel(const uint16_t* __restrict__ x0, float* __restrict__ out0,
                                                   Blocks blk0, const uint16_t* __restrict__ x1,
                                                   float* __restrict__ out1, Blocks blk1, int N) {
  constexpr int CH = D / 8;        // 16-byte chunks per row
  constexpr int RL = 256 / CH;     // row lanes
  __shared__ float red[RL][D + 4];

  const bool second = blockIdx.z == 1;
  const uint16_t* __restrict__ x = second ? x1 : x0;
  float* __restrict__ out = second ? out1 : out0;
  const Blocks& blk = second ? blk1 : blk0;
  const int i = blockIdx.x;
  if (i >= blk.nblocks) return;
  const int bh = blockIdx.y;
  int s, n;
  blk.get(bh, i, s, n);
  const int c = threadIdx.x % CH;
  const int r0 = threadIdx.x / CH;
  const uint16_t* xb = x + ((size_t)bh * N + s) * D + c * 8;

  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;

  int r = r0;
  // Four rows in flight per iteration.
  for (; r + 3 * RL < n; r += 4 * RL) {
    uint4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = *reinterpret_cast<const uint4*>(xb + (size_t)(r + u * RL) * D);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      acc[0] += bf16_lo(v[u].x); acc[1] += bf16_hi(v[u].x);
      acc[2] += bf16_lo(v[u].y); acc[3] += bf16_hi(v[u].y);
      acc[4] += bf16_lo(v[u].z); acc[5] += bf16_hi(v[u].z);
      acc[6] += bf16_lo(v[u].w); acc[7] += bf16_hi(v[u].w);
    }
  }
  for (; r < n; r += RL) {
    const uint4 v = *reinterpret_cast<const uint4*>(xb + (size_t)r * D);
    acc[0] += bf16_lo(v.x); acc[1] += bf16_hi(v.x);
    acc[2] += bf16_lo(v.y); acc[3] += bf16_hi(v.y);
    acc[4] += bf16_lo(v.z); acc[5] += bf16_hi(v.z);
    acc[6] += bf16_lo(v.w); acc[7] += bf16_hi(v.w);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[r0][c * 8 + e] = acc[e];
  __syncthreads();
  // Fixed-order tree over the row lanes.
#pragma unroll
  for (int h = RL / 2; h > 0; h >>= 1) {
    for (int t = threadIdx.x; t < h * D; t += 256) {
      const int rr = t / D, cc = t % D;
      red[rr][cc] += red[rr + h][cc];
    }
    __syncthreads();
  }
  if (threadIdx.x < D) {
    const float sum = red[0][threadIdx.x];
    out[((size_t)bh * blk.nblocks + i) * D + threadIdx.x] = n > 0 ? sum / (float)n : 0.f;
  }
}

hipError_t launch_pool(const uint16_t* x, int BH, int N, int d, const Blocks& blk, float* out,
                       hipStream_t s) {
  return launch_pool2(x, blk, out, nullptr, blk, nullptr, BH, N, d, s);
}

hipError_t launch_pool2(const uint16_t* x0, const Blocks& blk0, float* out0, const uint16_t* x1,
                        const Blocks& blk1, float* out1, int BH, int N, int d, hipStream_t s) {
  const int nb = x1 ? (blk0.nblocks > blk1.nblocks ? blk0.nblocks : blk1.nblocks) : blk0.nblocks;
  if (nb == 0 || BH == 0) return hipSuccess;
  dim3 grid(nb, BH, x1 ? 2 : 1);
  if (d == 128)
    pool_kernel<128><<<grid, 256, 0, s>>>(x0, out0, blk0, x1, out1, blk1, N);
  else
    pool_kernel<64><<<grid, 256, 0, s>>>(x0, out0, blk0, x1, out1, blk1, N);
  return hipGetLastError();
}

}  // namespace bsa
