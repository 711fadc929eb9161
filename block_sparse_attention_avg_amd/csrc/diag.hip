// Mask-quality diagnostic (Veda summary, section 2.1 "Punteggio dei Tile
// Distillato": the reference tile mask max-pools the full attention matrix
// over every query-tile x key-tile region, and a tile is described by the
// mean, maximum and minimum of its values; section 3 ties generation quality
// to how well a sparse mask matches that tile geometry). Like the pages'
// ground-truth heat maps it takes two passes: the full attention's row
// normalisers (the forward with every block kept and its row log-normaliser),
// then this pooled map.
//
// tile_stats_kernel: one 64-row query tile per workgroup (2 waves x 32 rows)
// walks every key tile of its head on double-buffered K tiles:
//   S^T = K Q^T (bf16 MFMA 32x32x16, Q^T in registers),
//   P = exp2(S * scale * log2e - lse * log2e),
// and reduces P over the tile's valid (query, key) pairs to its max, sum and
// min: lane-local, then a fixed butterfly over the wave, then the two waves'
// partials in LDS. Every order is fixed, so the map is bit-reproducible.
//
// check_mask_kernel: one wave per row of the lists; integer counts, so the
// totals are exact in any order.
//
// recall_kernel: one wave per (head, query block) row of the mask. The row's
// max-pooled values sit in LDS; a kept tile J is in the equal-budget oracle
// mask when fewer than k tiles outrank it (larger value, or equal value and a
// lower index), k being the row's kept count. The mass recall is the kept
// tiles' share of the row's attention mass.
#include "mfma_tile.h"

#include <math.h>

namespace bsa {

namespace {

__device__ __forceinline__ float wave_max_f(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_min_f(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fminf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum_f(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

}  // namespace

struct StatArgs {
  const uint16_t* q;
  const uint16_t* k;
  const float* lse;       // [BH][N] natural-log normaliser of the full attention rows
  float* tmax;            // [BH][nb][nb]
  float* tsum;
  float* tmin;
  int N, n_valid, nb;
  float scale;
};

template <int D>
__global__ __launch_bounds__(128) void tile_stats_kernel(StatArgs a, int BH) {
  using T = Tile<D>;
  constexpr int NS = D / 8;                        // MFMA steps of S^T
  __shared__ __align__(16) unsigned char K0[T::BYTES];
  __shared__ __align__(16) unsigned char K1[T::BYTES];
  __shared__ float part[2][2][3];                 // [chunk parity][wave][max, sum, min]

  // workgroups are dealt round-robin to the 8 XCDs; XCD x takes a contiguous
  // range of the (head, query tile) order so a head's K stays in one L2
  const int total = BH * a.nb, per = total >> 3, rem = total & 7;
  const int L = blockIdx.x, x = L & 7;
  const int p = x * per + min(x, rem) + (L >> 3);
  const int bh = p / a.nb, I = p - bh * a.nb;
  const int qs = 64 * I, ql = min(64, a.n_valid - qs);
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, half = lane >> 5, l32 = lane & 31;
  const size_t head = (size_t)bh * a.N;
  const uint16_t* kh = a.k + head * D;
  const float sl2 = a.scale * kLog2e;

  const int qr = 32 * wave + l32;
  const bool qok = qr < ql;
  bf16x8 qf[D / 16];
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    const size_t off = (head + qs + (qok ? qr : 0)) * D + 16 * c + 8 * half;
    qf[c] = qok ? *reinterpret_cast<const bf16x8*>(a.q + off) : bf16x8{};
  }
  const float lse2 = qok ? a.lse[head + qs + qr] * kLog2e : 0.f;
  float* omax = a.tmax + ((size_t)bh * a.nb + I) * a.nb;
  float* osum = a.tsum + ((size_t)bh * a.nb + I) * a.nb;
  float* omin = a.tmin + ((size_t)bh * a.nb + I) * a.nb;

  uint32_t off[T::NI];
  tile_offsets<D>(wave, lane, off);
  auto kl_of = [&](int J) { return min(64, a.n_valid - 64 * J); };

  // chunk J's two wave partials go out
  auto flush = [&](int J) {
    if (tid == 0) {
      const float(*pp)[3] = part[J & 1];
      omax[J] = fmaxf(pp[0][0], pp[1][0]);
      osum[J] = pp[0][1] + pp[1][1];
      omin[J] = fminf(pp[0][2], pp[1][2]);
    }
  };

  auto step = [&](int J, const lds_u8* Kc, lds_u8* Kn) {
    const int Jn = J + 1 < a.nb ? J + 1 : J;       // the last chunk reloads itself
    tile_load<D>(kh, 64 * Jn, kl_of(Jn), Kn, wave, off);
    wait_vm<T::NI>();                              // this wave's share of chunk J landed
    wg_barrier();                                  // and the other wave's
    if (J > 0) flush(J - 1);                       // (chunk J writes the other parity)
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const int kb = j & 1, cc = j >> 1;
      s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_read<D>(Kc, kb, cc, l32, half), qf[cc], s[kb], 0, 0, 0);
    }
    const int kl = kl_of(J);
    float mx = 0.f, sm = 0.f, mn = INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 32 * kb + acc_row(r, half);
        if (qok && key < kl) {
          const float pv = __builtin_amdgcn_exp2f(fmaf(s[kb][r], sl2, -lse2));
          mx = fmaxf(mx, pv);
          sm += pv;
          mn = fminf(mn, pv);
        }
      }
    mx = wave_max_f(mx);
    sm = wave_sum_f(sm);
    mn = wave_min_f(mn);
    if (lane == 0) {
      part[J & 1][wave][0] = mx;
      part[J & 1][wave][1] = sm;
      part[J & 1][wave][2] = mn;
    }
    wg_barrier();                                  // Kc free for chunk J+2; chunk J's partials complete
  };

  for (int J = 0;;) {
    if (J == 0) tile_load<D>(kh, 0, kl_of(0), (lds_u8*)K0, wave, off);
    step(J, (const lds_u8*)K0, (lds_u8*)K1);
    if (++J >= a.nb) break;
    step(J, (const lds_u8*)K1, (lds_u8*)K0);
    if (++J >= a.nb) break;
  }
  flush(a.nb - 1);
  wait_vm<0>();                                    // the last (repeated) load has landed
}

struct RecallArgs {
  const float* tmax;      // [rows][nkb]
  const float* tsum;
  const int32_t* kv_count;
  const int32_t* kv_index;
  int kv_stride, nkb;
  float* oracle_recall;   // [rows]
  float* mass_recall;
};

__global__ __launch_bounds__(256) void recall_kernel(RecallArgs a, size_t rows) {
  extern __shared__ float vals[];                  // [4][nkb]
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const size_t row = (size_t)blockIdx.x * 4 + wave;
  if (row >= rows) return;
  float* v = vals + (size_t)wave * a.nkb;
  const float* mx = a.tmax + row * a.nkb;
  const float* ms = a.tsum + row * a.nkb;
  float tot = 0.f;
  for (int j = lane; j < a.nkb; j += 64) {
    v[j] = mx[j];
    tot += ms[j];
  }
  tot = wave_sum_f(tot);
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (3 << 14));   // this wave's LDS writes are done
  __builtin_amdgcn_wave_barrier();
  const int cnt = min(max(a.kv_count[row], 0), a.kv_stride);
  const int32_t* list = a.kv_index + row * a.kv_stride;
  // the budget k: kept ids in range (an invalid id counts as not kept)
  int valid = 0;
  for (int e = lane; e < cnt; e += 64) valid += (unsigned)list[e] < (unsigned)a.nkb;
  valid = wave_sum_i(valid);
  float kept = 0.f;
  int hits = 0;
  for (int e = lane; e < cnt; e += 64) {
    const int J = list[e];
    if ((unsigned)J >= (unsigned)a.nkb) continue;
    kept += ms[J];
    const float x = v[J];
    int rank = 0;
    for (int j = 0; j < a.nkb; ++j) {
      const float y = v[j];
      rank += (y > x) || (y == x && j < J);
    }
    hits += rank < valid;
  }
  kept = wave_sum_f(kept);
  hits = wave_sum_i(hits);
  if (lane == 0) {
    a.oracle_recall[row] = valid > 0 ? (float)hits / (float)valid : 0.f;
    a.mass_recall[row] = tot > 0.f ? kept / tot : 0.f;
  }
}

__global__ __launch_bounds__(64) void zero_counts_kernel(int32_t* __restrict__ bad) {
  if (threadIdx.x < 3) bad[threadIdx.x] = 0;
}

// bad[0] += rows whose count lies outside [0, kv_stride]; for the other rows,
// over their first kv_count entries, bad[1] += ids outside [0, nkb) and
// bad[2] += ids not greater than the entry before them.
__global__ __launch_bounds__(256) void check_mask_kernel(const int32_t* __restrict__ kv_count,
                                                         const int32_t* __restrict__ kv_index, size_t rows, int nkb,
                                                         int kv_stride, int32_t* __restrict__ bad) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const size_t row = (size_t)blockIdx.x * 4 + wave;
  if (row >= rows) return;
  const int cnt = kv_count[row];
  if (cnt < 0 || cnt > kv_stride) {
    if (lane == 0) atomicAdd(&bad[0], 1);
    return;
  }
  const int32_t* l = kv_index + row * kv_stride;
  int oor = 0, uns = 0;
  for (int e = lane; e < cnt; e += 64) {
    const int v = l[e];
    oor += (unsigned)v >= (unsigned)nkb;
    uns += e > 0 && v <= l[e - 1];
  }
  oor = wave_sum_i(oor);
  uns = wave_sum_i(uns);
  if (lane == 0) {
    if (oor) atomicAdd(&bad[1], oor);
    if (uns) atomicAdd(&bad[2], uns);
  }
}

hipError_t launch_check_mask(const int32_t* kv_count, const int32_t* kv_index, size_t rows, int nkb, int kv_stride,
                             int32_t* bad, hipStream_t s) {
  zero_counts_kernel<<<1, 64, 0, s>>>(bad);
  if (rows > 0)
    check_mask_kernel<<<(unsigned)((rows + 3) / 4), 256, 0, s>>>(kv_count, kv_index, rows, nkb, kv_stride, bad);
  return hipGetLastError();
}

hipError_t launch_tile_stats(const uint16_t* q, const uint16_t* k, const float* lse, int BH, int N, int d,
                             int n_valid, float scale, float* tmax, float* tsum, float* tmin, hipStream_t s) {
  const int nb = (n_valid + 63) / 64;
  if (BH == 0 || nb == 0) return hipSuccess;
  StatArgs a{q, k, lse, tmax, tsum, tmin, N, n_valid, nb, scale};
  const unsigned grid = (unsigned)BH * nb;
  if (d == 128) tile_stats_kernel<128><<<grid, 128, 0, s>>>(a, BH);
  else tile_stats_kernel<64><<<grid, 128, 0, s>>>(a, BH);
  return hipGetLastError();
}

hipError_t launch_mask_recall(const float* tmax, const float* tsum, const int32_t* kv_count,
                              const int32_t* kv_index, int kv_stride, size_t rows, int nkb, float* oracle_recall,
                              float* mass_recall, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  RecallArgs a{tmax, tsum, kv_count, kv_index, kv_stride, nkb, oracle_recall, mass_recall};
  const size_t lds = sizeof(float) * 4 * (size_t)nkb;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(recall_kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  recall_kernel<<<(unsigned)((rows + 3) / 4), 256, lds, s>>>(a, rows);
  return hipGetLastError();
}

}  // namespace bsa
